"""Oracle parity of EVERY output at the full sizes of the measured workloads,
and of the softmax regimes the flat N(0, 1) workloads never reach.

Full sizes, in the launch configuration bench.py times (library-default
splits unless stated), every live request x every query head x every head
dim against the fp64 oracle, and the pool pages of every live request byte
for byte:
  gqa8_16k_b64        64 x 16384 tokens, e4m3, 2 GiB pool; also through the
                      append taken into the attention launch
  gqa8_16k_b32        the bf16 twin, 32 x 16384 tokens in the same 2 GiB
  gqa8_16k_b{1,8,16}  the small concurrency points, e4m3 and bf16
  mha_g1_16k_b8       8 x 16384 tokens, 32 query heads = 32 KV heads, both
                      pools, one split and 8 (wave-per-split mode)
  gqa8_256k_b4        4 x 262144 tokens, one stale request, at the stated 64
                      splits and at the library default

Peaked softmax and dynamic range (device-drawn, seeded; inputs.py recipes):
  q x16 and x64 (scores spanning tens to hundreds of nats, many running-max
  rescales), V with a biased channel mean (+4 on even head dims), K and V
  data scaled by 2^+-20 (scales amax/448 far from 1, with q scaled the other
  way so the scores stay peaked; outputs compared after undoing the V
  factor), for S = 1, S = 4 and the balanced partition, both pool types, on
  the BIG-page MFMA path, the 16-token-page path (G = 4) and one query head
  per KV head (G = 1); and the needle case at 262144 tokens: every wave's first tile holds
  a needle and the other 262,000 tokens each weigh about exp(-17.6) of one,
  below half of fp16's smallest subnormal, so a kernel that rounded P to fp16
  would drop their 0.07% of the mass (x the +4 channel bias: 3e-3 absolute)
  from the numerator while keeping it in the denominator.

Bar: |gpu - oracle| <= 2e-3 + 1e-2 |oracle| for out and lse, element-wise.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from paged_attention_fp8_amd import harness as H
from paged_attention_fp8_amd import inputs as I
from paged_attention_fp8_amd import ops
from helpers import allclose_report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ATOL, RTOL = 2e-3, 1e-2


def say(*a):
    print(*a, flush=True)


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_status(inp):
    return oracle.page_tag_check(inp.batch.page_table, inp.batch.context_lens,
                                 inp.batch.expected_tags, inp.pool.tags, inp.workload.page_size)


def full_oracle(inp, kv_dtype):
    """The oracle's pool (every token of every request the oracle's own check
    passes, quantised by the oracle from the same bf16 source) and its
    outputs for every request and head."""
    w = inp.workload
    status = oracle_status(inp)
    fill = H.FP8_NAN_CODE if kv_dtype == oracle.KV_FP8 else H.BF16_NAN_BITS
    pool = oracle.Pool(kv_dtype, inp.num_pages, w.kv_heads, w.page_size, w.head_dim, fill=fill)
    table, lens = inp.batch.page_table, inp.batch.context_lens
    ks = inp.k_scale if kv_dtype == oracle.KV_FP8 else None
    vs = inp.v_scale if kv_dtype == oracle.KV_FP8 else None
    B = inp.batch.batch
    chunk = 16   # bounds the host copy of the bf16 source
    for b0 in range(0, B, chunk):
        b1 = min(B, b0 + chunk)
        T = int(lens[b0:b1].max())
        k = host_bits(inp.k_tokens[b0:b1, :T])
        v = host_bits(inp.v_tokens[b0:b1, :T])
        oracle.kv_write(pool, table[b0:b1], np.zeros(b1 - b0, np.int32), lens[b0:b1], k, v, ks, vs,
                        status=status[b0:b1])
        del k, v
    ro, rl = oracle.paged_attention(pool, host_bits(inp.q), table, lens,
                                    1.0 / math.sqrt(w.head_dim), ks, vs, status=status)
    return pool, ro, rl, status


def pools_match(step, inp, pool, status, kv_dtype):
    gk, gv = step.cache.k_pool.cpu(), step.cache.v_pool.cpu()
    if kv_dtype == ops.KV_BF16:
        gk = gk.view(torch.int16).numpy().view(np.uint16)
        gv = gv.view(torch.int16).numpy().view(np.uint16)
    else:
        gk, gv = gk.numpy(), gv.numpy()
    P = inp.workload.page_size
    live = [b for b in range(inp.batch.batch) if status[b] == 0]
    pages = np.concatenate([inp.batch.page_table[b][:I.pages_needed(inp.batch.context_lens[b], P)]
                            for b in live]) if live else np.zeros(0, np.int64)
    assert np.array_equal(gk[pages], pool.k[pages]), "K pages differ from the oracle's"
    assert np.array_equal(gv[pages], pool.v[pages]), "V pages differ from the oracle's"
    say(f"  pools: {len(pages)} pages of {len(live)} live requests byte-exact")


def compare_all(out, lse, ro, rl, what, out_factor=1.0, status=None):
    """Every element of out and lse of the live requests (aborted ones are
    checked exactly by check_aborted); out_factor undoes a power-of-two V
    scale (exact) so that the tolerance applies at the data's own magnitude."""
    live = np.ones(out.shape[0], bool) if status is None else np.asarray(status) == 0
    o = out.cpu().numpy()[live].astype(np.float64) * out_factor
    ok1, ma, mr = allclose_report(o, ro[live] * out_factor, ATOL, RTOL)
    ok2, la, lr = allclose_report(lse.cpu().numpy()[live], rl[live], ATOL, RTOL)
    say(f"  {what}: {o.size} outputs, out max_abs={ma:.3e} max_rel={mr:.3e}; "
        f"lse max_abs={la:.3e}")
    assert ok1 and ok2, f"{what}: out max_abs={ma} rel={mr}, lse max_abs={la} rel={lr}"


def check_aborted(out, lse, status):
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for b in np.nonzero(status)[0]:
        assert np.all(o[b] == 0) and np.all(np.isneginf(l[b])), f"aborted request {b}"


# ---------------------------------------------------------------------------
# full sizes
# ---------------------------------------------------------------------------

def test_b64_e4m3_every_output_and_append_in_launch():
    """64 x 16k e4m3 (the headline point), library-default splits: every
    output, every pool page; first through the append taken into the
    attention launch (the pool then holds only the history before the call),
    then through the separate append + attention calls."""
    w = I.WORKLOADS["gqa8_16k_b64"]
    say(f"workload {w.name}")
    inp = I.make_device_decode_inputs(w, 1003, DEV)
    pool, ro, rl, status = full_oracle(inp, oracle.KV_FP8)
    step = H.build_step(inp, ops.KV_FP8_E4M3, DEV, poison=True)
    sm = 1.0 / math.sqrt(w.head_dim)
    out, lse, st = H.decode_step(step, sm, 0, append_in_attention=True)
    torch.cuda.synchronize()
    assert np.array_equal(st.cpu().numpy(), status)
    pools_match(step, inp, pool, status, ops.KV_FP8_E4M3)
    compare_all(out, lse, ro, rl, "append in the attention launch")
    out, lse, st = H.decode_step(step, sm, 0)
    torch.cuda.synchronize()
    pools_match(step, inp, pool, status, ops.KV_FP8_E4M3)
    compare_all(out, lse, ro, rl, "check + append + attention")


def test_b32_bf16_twin_every_output():
    w = I.sweep_workload(32, 2)
    say(f"workload {w.name} bf16")
    inp = I.make_device_decode_inputs(w, 1004, DEV)
    pool, ro, rl, status = full_oracle(inp, oracle.KV_BF16)
    step = H.build_step(inp, ops.KV_BF16, DEV, poison=True)
    out, lse, st = H.decode_step(step, 1.0 / math.sqrt(w.head_dim), 0)
    torch.cuda.synchronize()
    pools_match(step, inp, pool, status, ops.KV_BF16)
    compare_all(out, lse, ro, rl, "bf16 twin")


@pytest.mark.parametrize("kv_dtype", [ops.KV_FP8_E4M3, ops.KV_BF16], ids=["fp8", "bf16"])
@pytest.mark.parametrize("batch", [1, 8, 16])
def test_small_concurrency_points_every_output(batch, kv_dtype):
    """The concurrency points below 32 requests run with split-K by default
    (16, 4 and 2 splits at 1, 8 and 16 requests on 256 CUs): every output,
    through both the separate append and the append inside the launch."""
    w = I.sweep_workload(batch, 1 if kv_dtype == ops.KV_FP8_E4M3 else 2)
    say(f"workload {w.name} dtype={kv_dtype}")
    inp = I.make_device_decode_inputs(w, 1010 + batch, DEV)
    pool, ro, rl, status = full_oracle(inp, kv_dtype)
    sm = 1.0 / math.sqrt(w.head_dim)
    for fused in (True, False):
        step = H.build_step(inp, kv_dtype, DEV, poison=True)
        out, lse, _ = H.decode_step(step, sm, 0, append_in_attention=fused)
        torch.cuda.synchronize()
        pools_match(step, inp, pool, status, kv_dtype)
        compare_all(out, lse, ro, rl, f"default splits ({'append in launch' if fused else 'separate'})")
        del step


@pytest.mark.parametrize("kv_dtype", [ops.KV_FP8_E4M3, ops.KV_BF16], ids=["fp8", "bf16"])
def test_one_query_head_per_kv_head_every_output(kv_dtype):
    """The bench's one-query-head-per-KV-head workload (8 x 16k tokens, 32
    heads, a group of one on the MFMA kernels): every output at the library
    default (one split) and at 8 splits, which on 256 CUs runs the
    wave-per-split mode (2048 splits, two per wave)."""
    w = I.Workload("mha_g1_16k_b8", 8, 32, 32, 128, 64, 16384, 16384, pool_factor=1.0)
    say(f"workload {w.name} dtype={kv_dtype}")
    inp = I.make_device_decode_inputs(w, 1020, DEV)
    pool, ro, rl, status = full_oracle(inp, kv_dtype)
    step = H.build_step(inp, kv_dtype, DEV, poison=True)
    sm = 1.0 / math.sqrt(w.head_dim)
    for splits in (0, 8):
        out, lse, _ = H.decode_step(step, sm, splits)
        torch.cuda.synchronize()
        compare_all(out, lse, ro, rl, f"splits={splits or 'default'}")
    pools_match(step, inp, pool, status, kv_dtype)


def test_long_context_256k_every_live_output():
    """4 x 262144 tokens with one stale request: the check aborts exactly it
    (out 0, lse -inf); every output of the 3 live requests at the stated 64
    splits and at the library default."""
    w = I.WORKLOADS["gqa8_256k_b4"]
    say(f"workload {w.name}")
    inp = I.make_device_decode_inputs(w, 1005, DEV)
    pool, ro, rl, status = full_oracle(inp, oracle.KV_FP8)
    assert int((status != 0).sum()) == 1
    step = H.build_step(inp, ops.KV_FP8_E4M3, DEV, poison=True)
    sm = 1.0 / math.sqrt(w.head_dim)
    for splits in (w.num_splits, 0):
        out, lse, st = H.decode_step(step, sm, splits)
        torch.cuda.synchronize()
        assert np.array_equal(st.cpu().numpy(), status)
        check_aborted(out, lse, status)
        compare_all(out, lse, ro, rl, f"splits={splits or 'default'}", status=status)
    pools_match(step, inp, pool, status, ops.KV_FP8_E4M3)


# ---------------------------------------------------------------------------
# peaked softmax, biased V, extreme scales
# ---------------------------------------------------------------------------

def _w(name, B, Hq, Hkv, P, L, **kw):
    return I.Workload(name, B, Hq, Hkv, 128, P, L, L, pool_factor=1.25, **kw)


PEAKED = [
    _w("q16_vbias_16k", 2, 64, 8, 64, 16384, q_mult=16.0, v_bias=4.0),
    _w("q64_vbias_16k", 2, 64, 8, 64, 16384, q_mult=64.0, v_bias=4.0),
    # K data x 2^20 (k_scale ~ 2^20 amax/448), q x 64 x 2^-20, V data x 2^-20
    _w("q64_k+20_v-20_16k", 2, 64, 8, 64, 16384, q_mult=64.0 * 2.0 ** -20, k_log2=20, v_log2=-20,
       v_bias=4.0),
    # K data x 2^-20, q x 16 x 2^20, V data x 2^20
    _w("q16_k-20_v+20_16k", 2, 64, 8, 64, 16384, q_mult=16.0 * 2.0 ** 20, k_log2=-20, v_log2=20,
       v_bias=4.0),
    # 16-token pages (the page-gathering MFMA path), G = 4
    _w("q16_vbias_gqa4_p16_8k", 2, 32, 8, 16, 8192, q_mult=16.0, v_bias=4.0),
    # one query head per KV head (one live MFMA column)
    _w("q16_vbias_mha_16k", 1, 8, 8, 64, 16384, q_mult=16.0, v_bias=4.0),
]


@pytest.mark.parametrize("kv_dtype", [ops.KV_FP8_E4M3, ops.KV_BF16], ids=["fp8", "bf16"])
@pytest.mark.parametrize("w", PEAKED, ids=lambda w: w.name)
def test_peaked_softmax_and_extreme_scales(w, kv_dtype):
    say(f"peaked: {w.name} dtype={kv_dtype}")
    inp = I.make_device_decode_inputs(w, 1100, DEV)
    pool, ro, rl, status = full_oracle(inp, kv_dtype)
    # the regime is the intended one: the softmax is far from flat
    spread = float(np.max(rl) - np.min(rl))
    say(f"  lse range {np.min(rl):.1f} .. {np.max(rl):.1f}")
    assert spread > 20.0 or np.max(np.abs(rl)) > 20.0
    step = H.build_step(inp, kv_dtype, DEV, poison=True)
    sm = 1.0 / math.sqrt(w.head_dim)
    factor = 2.0 ** -w.v_log2
    for splits in (1, 4, ops.BALANCED):
        out, lse, _ = H.decode_step(step, sm, splits)
        torch.cuda.synchronize()
        compare_all(out, lse, ro, rl, f"splits={splits}", out_factor=factor)
    pools_match(step, inp, pool, status, kv_dtype)


@pytest.mark.parametrize("kv_dtype", [ops.KV_FP8_E4M3, ops.KV_BF16], ids=["fp8", "bf16"])
def test_needle_262144_tokens(kv_dtype):
    """One request of 262144 tokens whose needles score 17.6 nats above a
    flat background, V biased +4 on even head dims: at S = 1 every wave meets
    a needle in its first tile, so all later weights are about 2^-25.4."""
    w = I.Workload("needle_256k", 1, 64, 8, 128, 64, 262144, 262144, pool_factor=1.0,
                   needle_gap=17.6, v_bias=4.0)
    say(f"needle: {w.name} dtype={kv_dtype}")
    inp = I.make_device_decode_inputs(w, 1200, DEV)
    pool, ro, rl, status = full_oracle(inp, kv_dtype)
    step = H.build_step(inp, kv_dtype, DEV, poison=True)
    sm = 1.0 / math.sqrt(w.head_dim)
    for splits in (1, 0, ops.BALANCED):
        out, lse, _ = H.decode_step(step, sm, splits)
        torch.cuda.synchronize()
        compare_all(out, lse, ro, rl, f"splits={splits}")


# ---------------------------------------------------------------------------
# the _append entry points against the oracle at small sizes
# ---------------------------------------------------------------------------

APPEND_CASES = [
    I.Workload("mha_d64_p16", 3, 4, 4, 64, 16, 1, 300, pool_factor=1.5),
    I.Workload("gqa4_d128_p16", 3, 16, 4, 128, 16, 250, 1100, pool_factor=1.3),
    I.Workload("gqa8_d128_p64", 4, 16, 2, 128, 64, 1, 1500, pool_factor=1.3),
    I.Workload("gqa16_d64_p32", 2, 32, 2, 64, 32, 300, 900, pool_factor=1.3),
]


@pytest.mark.parametrize("splits", [1, 3, ops.BALANCED], ids=["S1", "S3", "balanced"])
@pytest.mark.parametrize("kv_dtype", [ops.KV_FP8_E4M3, ops.KV_BF16], ids=["fp8", "bf16"])
@pytest.mark.parametrize("w", APPEND_CASES, ids=lambda w: w.name)
def test_append_entry_points_match_oracle(w, kv_dtype, splits):
    """paged_decode_attn_{fp8,bf16}_append: pools byte-exact and outputs
    within tolerance of the oracle's check + append + attention, one stale
    request aborted (seeds other than the attention tests')."""
    say(f"append entry: {w.name} dtype={kv_dtype} splits={splits}")
    wl = I.scaled(w, stale_requests=1 if w.batch > 2 else 0)
    inp = I.make_device_decode_inputs(wl, 77, DEV)
    pool, ro, rl, status = full_oracle(inp, kv_dtype)
    step = H.build_step(inp, kv_dtype, DEV, poison=True)
    out, lse, st = H.decode_step(step, 1.0 / math.sqrt(w.head_dim), splits, append_in_attention=True)
    torch.cuda.synchronize()
    assert np.array_equal(st.cpu().numpy(), status)
    pools_match(step, inp, pool, status, kv_dtype)
    check_aborted(out, lse, status)
    compare_all(out, lse, ro, rl, "append entry point", status=status)
