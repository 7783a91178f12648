"""INT4 weight streaming on the GPU (int4_pack_weights, int4_gemv) against
the oracle.  Tolerance (the bound include/pafp8.h states): products are
exact and summed in fp32, 128 per group and then over the groups, so
    |y - exact| <= (K/128 + 160) * 2^-24 * sum_k |x| (|q| + c) s,
with c = 272 for rows computed by a launch of at most 16 rows, or of 17 to
32 rows when K is not a multiple of 1024 (those paths sum x (136 + q) and
take 136 sum x back out), and c = 0 otherwise, checked with a factor 2 of
slack."""
import numpy as np
import pytest
import torch

import oracle
from paged_attention_fp8_amd import inputs as I
from paged_attention_fp8_amd import ops
from helpers import int4_blocks, int4_rowmajor

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def _dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(DEV)


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).to(DEV).view(torch.bfloat16)


def _case(M, N, K, seed):
    g = np.random.default_rng(seed)
    q = g.integers(-8, 8, (N, K)).astype(np.int8)
    q[0, :8] = [-8, -8, 7, 7, 0, -1, 1, -8]               # the extremes, in one dword
    xf = g.standard_normal((M, K)).astype(np.float32)
    xf[g.random((M, K)) < 0.01] *= 30.0                    # outliers
    x = I.f32_to_bf16_bits(xf)
    s = I.f32_to_bf16_bits((g.random((K // 128, N)) * 0.05 + 1e-4).astype(np.float32))
    return q, x, s


def _bound(q, x, s):
    N, K = q.shape
    M = x.shape[0]
    # rows go to launches of 64; a launch of at most 16 rows, or of 17 to 32
    # rows with K not a multiple of 1024, adds c = 272
    launch_rows = np.where(np.arange(M) < M // 64 * 64, 64, M % 64)
    plus136 = (launch_rows <= 16) | ((launch_rows <= 32) & (K % 1024 != 0))
    off_rows = np.where(plus136, 272.0, 0.0)
    xa = np.abs(I.bf16_bits_to_f32(x).astype(np.float64))
    sf = I.bf16_bits_to_f32(s).astype(np.float64)
    out = np.empty((M, N))
    for off in np.unique(off_rows):
        rows = off_rows == off
        for n0 in range(0, N, 1024):             # rows in chunks: bounded memory
            wa = (np.abs(q[n0:n0 + 1024].astype(np.float64)) + off) * np.repeat(sf[:, n0:n0 + 1024], 128, axis=0).T
            out[rows, n0:n0 + 1024] = xa[rows] @ wa.T
    return 2.0 * (K / 128 + 160) * 2.0 ** -24 * out


def test_pack_matches_documented_layout():
    say("int4: pack kernel vs NumPy layout")
    for N, K in [(16, 512), (48, 1024), (128, 4096)]:
        q, _, _ = _case(1, N, K, N + K)
        packed = ops.int4_pack_weights(_dev_u8(int4_rowmajor(q)), N, K).cpu().numpy()
        assert np.array_equal(packed, int4_blocks(q)), (N, K)


@pytest.mark.parametrize("M,N,K", [(1, 16, 512), (2, 48, 1536), (1, 1008, 2048), (5, 48, 512),
                                   (16, 64, 1024), (17, 80, 1536), (33, 128, 512), (64, 256, 2048),
                                   (100, 32, 512), (66, 32, 512), (3, 1008, 1024)])
def test_gemv_matches_oracle(M, N, K):
    say(f"int4 gemv: M={M} N={N} K={K}")
    q, x, s = _case(M, N, K, M * 1000 + N + K)
    packed = int4_blocks(q)
    y = ops.int4_gemv(_dev_bf16(x), _dev_u8(packed), _dev_bf16(s), N, K).cpu().numpy()
    ref = oracle.int4_gemv(x, packed, s, N, K)
    err = np.abs(y - ref)
    bound = _bound(q, x, s)
    assert np.all(err <= bound), (err.max(), bound[err > bound][:4])


def test_gemv_full_size_decode_shape():
    """The measured shape (28672 x 8192): at one row every output against the
    oracle; at 32 and 64 rows, 16 sampled 16-row tiles of the output."""
    N, K = 28672, 8192
    for M in (1, 2, 32, 64):
        say(f"int4 gemv full size: M={M}")
        q, x, s = _case(M, N, K, 99 + M)
        packed = ops.int4_pack_weights(_dev_u8(int4_rowmajor(q)), N, K)
        y = ops.int4_gemv(_dev_bf16(x), packed, _dev_bf16(s), N, K).cpu().numpy()
        if M <= 2:
            rows = np.arange(N)
        else:
            tiles = np.random.default_rng(5).choice(N // 16, 16, replace=False)
            rows = (tiles[:, None] * 16 + np.arange(16)).reshape(-1)
        qs, ss = q[rows], np.ascontiguousarray(s[:, rows])
        ref = oracle.int4_gemv(x, int4_blocks(qs), ss, len(rows), K)
        err = np.abs(y[:, rows] - ref)
        bound = _bound(qs, x, ss)
        assert np.all(err <= bound), (err.max(), (err / bound).max())


@pytest.mark.parametrize("M,N,K", [(8, 20480, 1536), (16, 24576, 1024), (2, 28688, 2048),
                                   (16, 32768, 512), (9, 28672, 1536)])
def test_gemv_tiles_per_work_group(M, N, K):
    """2-16 rows with the tile count per work-group chosen from the CU count
    (on 256 CUs: 5, 6, 8 with a last work-group holding one live tile, 8,
    and 7), both prefetch depths: every output within the bound."""
    say(f"int4 gemv tiles per work-group: M={M} N={N} K={K}")
    q, x, s = _case(M, N, K, 31 * M + N + K)
    packed = int4_blocks(q)
    y = ops.int4_gemv(_dev_bf16(x), _dev_u8(packed), _dev_bf16(s), N, K).cpu().numpy()
    ref = oracle.int4_gemv(x, packed, s, N, K)
    err = np.abs(y - ref)
    bound = _bound(q, x, s)
    assert np.all(err <= bound), (err.max(), (err / bound).max())


def test_gemv_edges():
    say("int4 gemv: empty and invalid shapes")
    x = torch.zeros((0, 512), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(16 * 512 // 2, dtype=torch.uint8, device=DEV)
    sc = torch.zeros((4, 16), dtype=torch.bfloat16, device=DEV)
    assert ops.int4_gemv(x, w, sc, 16, 512).shape == (0, 16)
    with pytest.raises(ops.Pafp8Error, match="K of 512"):
        ops.int4_gemv(torch.zeros((1, 384), dtype=torch.bfloat16, device=DEV),
                      torch.zeros(16 * 384 // 2, dtype=torch.uint8, device=DEV),
                      torch.zeros((3, 16), dtype=torch.bfloat16, device=DEV), 16, 384)


def _random_shapes(n, seed=2028):
    g = np.random.default_rng(seed)
    return [(int(g.integers(1, 81)), 16 * int(g.integers(1, 65)), 512 * int(g.integers(1, 9)))
            for _ in range(n)]


@pytest.mark.parametrize("M,N,K", _random_shapes(20))
def test_gemv_random_shapes(M, N, K):
    """Seeded random shapes (every launch path: 1 row, 2-32, 33-64, more than
    64 rows), within the stated bound of the oracle."""
    say(f"int4 gemv random: M={M} N={N} K={K}")
    q, x, s = _case(M, N, K, 7 * M + 3 * N + K)
    packed = int4_blocks(q)
    y = ops.int4_gemv(_dev_bf16(x), _dev_u8(packed), _dev_bf16(s), N, K).cpu().numpy()
    ref = oracle.int4_gemv(x, packed, s, N, K)
    err = np.abs(y - ref)
    bound = _bound(q, x, s)
    assert np.all(err <= bound), (err.max(), (err / bound).max())
