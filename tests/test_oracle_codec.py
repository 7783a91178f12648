"""Pins for the oracle's e4m3 codec (decode O1, encode O2, quantise O4).

Each check ties the oracle to something other than itself: hand-worked
anchors from the format definition (tests/golden), torch's independent
float8_e4m3fn implementation, the brute-force nearest-code search, and
structural invariants of the format.  The pages name the format only as
"FP8 (e4m3)" (Cloudflare, "Smaller, faster, safer: running Kimi and GLM at
scale", section "KV 缓存量化" / KV cache quantization).
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_pairs(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()[:2]
            rows.append((a, b))
    return rows


def _torch_decode_all():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_golden_anchors(oracle_mod):
    for code, val in _read_pairs("e4m3_decode_anchors.txt"):
        got = oracle_mod.e4m3_decode(int(code, 16))
        want = float(val)
        if math.isnan(want):
            assert math.isnan(got), code
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)


def test_decode_matches_torch_for_all_codes(oracle_mod):
    ours = oracle_mod.e4m3_decode_table()
    ref = _torch_decode_all()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_decode_structure(oracle_mod):
    t = oracle_mod.e4m3_decode_table()
    fin = ~np.isnan(t)
    assert fin.sum() == 254
    assert [c for c in range(256) if np.isnan(t[c])] == [0x7F, 0xFF]
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # strictly increasing magnitudes
    assert np.array_equal(t[0x80:0xFF], -pos)            # sign-magnitude
    assert pos.max() == 448.0 and pos[1] == 2.0 ** -9 and pos[8] == 2.0 ** -6
    # every finite value is exact in bf16 and in fp16 (decode-on-read may use either)
    v = t[fin]
    assert np.array_equal(v.astype(np.float16).astype(np.float64), v)
    bf = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf, v)


def test_encode_golden_anchors(oracle_mod):
    for val, code in _read_pairs("e4m3_encode_anchors.txt"):
        x = np.float32(float(val))
        assert oracle_mod.e4m3_encode([x])[0] == int(code, 16), val
        assert oracle_mod.e4m3_encode_brute([x])[0] == int(code, 16), val


def _boundary_values(oracle_mod):
    """Every code value, every midpoint between neighbours, and their fp32
    neighbours one ulp away, with both signs."""
    t = oracle_mod.e4m3_decode_table()[:0x7F]
    mids = (t[:-1] + t[1:]) / 2
    base = np.concatenate([t, mids, [448.0, 464.0, 480.0, 1e4]]).astype(np.float32)
    up = np.nextafter(base, np.float32(np.inf))
    dn = np.nextafter(base, np.float32(-np.inf))
    v = np.concatenate([base, up, dn])
    return np.concatenate([v, -v]).astype(np.float32)


def test_encode_fast_equals_brute_on_boundaries(oracle_mod):
    v = _boundary_values(oracle_mod)
    assert np.array_equal(oracle_mod.e4m3_encode(v), oracle_mod.e4m3_encode_brute(v))


def test_encode_fast_equals_brute_random(oracle_mod):
    g = np.random.default_rng(7)
    n = 400_000
    mag = np.exp2(g.uniform(-14, 10, n)).astype(np.float32)
    sign = np.where(g.random(n) < 0.5, -1, 1).astype(np.float32)
    raw = g.integers(0, 2 ** 32, 20_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    v = np.concatenate([mag * sign, raw])
    assert np.array_equal(oracle_mod.e4m3_encode(v), oracle_mod.e4m3_encode_brute(v))


def test_encode_matches_torch_below_saturation(oracle_mod):
    # torch rounds to nearest-even but turns |x| >= 464 into NaN instead of
    # saturating; below that the two definitions coincide
    g = np.random.default_rng(11)
    n = 4_000_000
    mag = np.exp2(g.uniform(-20, np.log2(463.9), n)).astype(np.float32)
    v = np.concatenate([mag, -mag, _boundary_values(oracle_mod)])
    v = v[np.abs(v) < 464.0]
    assert np.array_equal(oracle_mod.e4m3_encode(v), _torch_encode(v))


def test_encode_round_trip_and_monotone(oracle_mod):
    t = oracle_mod.e4m3_decode_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])])
    assert np.array_equal(oracle_mod.e4m3_encode(t[codes].astype(np.float32)), codes)
    g = np.random.default_rng(3)
    v = np.sort(g.uniform(-500, 500, 200_000).astype(np.float32))
    dec = t[oracle_mod.e4m3_encode(v)]
    assert np.all(np.diff(dec) >= 0)


def test_encode_all_fp32_patterns_sampled_against_torch(oracle_mod):
    # a strided walk over the whole 2^32 bit-pattern space, compared where
    # torch's definition applies (finite, |x| < 464)
    first, n = 0x00000123, 1 << 22
    bits = (np.arange(n, dtype=np.uint64) * 1021 + first).astype(np.uint32)
    x = bits.view(np.float32)
    ours = oracle_mod.e4m3_encode(x)
    ok = np.isfinite(x) & (np.abs(x) < 464.0)
    assert np.array_equal(ours[ok], _torch_encode(x[ok]))
    big = np.isfinite(x) & (np.abs(x) >= 448.0)
    assert np.all(ours[big] == np.where(np.signbit(x[big]), 0xFE, 0x7E))
    nan = np.isnan(x)
    assert np.all(ours[nan] == np.where(np.signbit(x[nan]), 0xFF, 0x7F))


def test_bits_range_matches_array_form(oracle_mod):
    first = 0x3F7FF000
    n = 8192
    x = (np.arange(n, dtype=np.uint64) + first).astype(np.uint32).view(np.float32)
    assert np.array_equal(oracle_mod.e4m3_encode_bits_range(first, n), oracle_mod.e4m3_encode(x))


def test_quantize_uses_fp32_division(oracle_mod):
    """quantise(x, s) == e4m3(f32(x) / s), with the division an IEEE single
    division (numpy's float32 divide) and the encode torch's."""
    from paged_attention_fp8_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits
    g = np.random.default_rng(5)
    xs = f32_to_bf16_bits(g.standard_normal(20_000).astype(np.float32) * 3)
    ss = (np.abs(g.standard_normal(20_000)) * 0.02 + 1e-3).astype(np.float32)
    q = bf16_bits_to_f32(xs) / ss
    keep = np.abs(q) < 464.0
    want = _torch_encode(q[keep])
    got = np.array([oracle_mod.quantize(int(x), float(s)) for x, s in zip(xs[keep], ss[keep])],
                   dtype=np.uint8)
    assert np.array_equal(got, want)


def test_quantize_closed_forms(oracle_mod):
    from paged_attention_fp8_amd.inputs import f32_to_bf16_bits
    amax = np.float32(5.25)
    s = float(np.float32(amax) / np.float32(448.0))
    one = lambda v: int(f32_to_bf16_bits(np.array([v], np.float32))[0])
    assert oracle_mod.quantize(one(5.25), s) == 0x7E       # amax maps onto 448
    assert oracle_mod.quantize(one(-5.25), s) == 0xFE
    assert oracle_mod.quantize(one(0.0), s) == 0x00
    assert oracle_mod.quantize(one(-0.0), s) == 0x80
    assert oracle_mod.quantize(one(105.0), s) == 0x7E      # x20 outlier saturates
    assert oracle_mod.quantize(one(1.0), 1.0) == 0x38


@pytest.mark.parametrize("scale", [1.0, 0.0123, 3.5])
def test_quantize_equals_encode_of_quotient(oracle_mod, scale):
    from paged_attention_fp8_amd.inputs import bf16_bits_to_f32
    xs = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore", over="ignore"):   # NaN stays NaN; large values overflow to inf
        q = bf16_bits_to_f32(xs) / np.float32(scale)
    want = oracle_mod.e4m3_encode(q)
    got = np.array([oracle_mod.quantize(int(x), scale) for x in xs], np.uint8)
    assert np.array_equal(got, want)
