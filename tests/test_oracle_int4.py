"""Pins of the oracle's INT4 weight-streaming product (oracle_int4_gemv,
oracle_int4_unpack) against things other than itself: the packed layout
written out in NumPy, float64 NumPy matrix products, and closed forms."""
import numpy as np
import pytest

import oracle
from paged_attention_fp8_amd import inputs as I
from helpers import int4_blocks, int4_rowmajor


def _case(M, N, K, seed):
    g = np.random.default_rng(seed)
    q = g.integers(-8, 8, (N, K)).astype(np.int8)
    x = I.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    s = I.f32_to_bf16_bits((g.random((K // 128, N)) * 0.05 + 1e-3).astype(np.float32))
    return q, x, s


def _f64(bits):
    return I.bf16_bits_to_f32(bits).astype(np.float64)


def test_unpack_inverts_the_numpy_layout():
    q, _, _ = _case(1, 48, 1024, 1)
    assert np.array_equal(oracle.int4_unpack(int4_blocks(q), 48, 1024), q)


def test_rowmajor_nibbles():
    q = np.array([[0, 1, -1, 7, -8, 3, 2, -2]], np.int8)
    assert int4_rowmajor(q).tolist() == [[0x10, 0x7F, 0x38, 0xE2]]


@pytest.mark.parametrize("M,N,K", [(1, 16, 512), (5, 48, 1024), (64, 32, 512), (3, 16, 2048)])
def test_gemv_equals_numpy_float64(M, N, K):
    q, x, s = _case(M, N, K, M * 7 + N)
    y = oracle.int4_gemv(x, int4_blocks(q), s, N, K)
    w = q.astype(np.float64) * np.repeat(_f64(s), 128, axis=0).T   # [N][K]
    ref = _f64(x) @ w.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_closed_forms():
    N, K = 32, 512
    q, _, s = _case(1, N, K, 3)
    packed = int4_blocks(q)
    # one-hot activations pick one weight times its scale
    for k in (0, 1, 127, 128, 300, 511):
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        y = oracle.int4_gemv(I.f32_to_bf16_bits(x), packed, s, N, K)
        assert np.array_equal(y[0], q[:, k] * _f64(s)[k // 128])
    # all-ones weights and unit scales give the row sums of x; -8 is negative
    ones = np.ones((N, K), np.int8)
    unit = I.f32_to_bf16_bits(np.ones((K // 128, N), np.float32))
    _, x, _ = _case(2, N, K, 4)
    y = oracle.int4_gemv(x, int4_blocks(ones), unit, N, K)
    assert np.allclose(y, _f64(x).sum(1)[:, None] * np.ones(N), rtol=1e-12)
    eights = np.full((N, K), -8, np.int8)
    y = oracle.int4_gemv(x, int4_blocks(eights), unit, N, K)
    assert np.allclose(y, -8 * _f64(x).sum(1)[:, None] * np.ones(N), rtol=1e-12)
