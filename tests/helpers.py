"""Test-side helpers: oracle-side cache construction and an independent
NumPy/torch textbook attention used to pin the oracle.

Nothing here touches the HIP library.
"""
import numpy as np
import torch
from scipy.special import logsumexp

import oracle
from paged_attention_fp8_amd import inputs as I

FP8_NAN = 0x7F
BF16_NAN = 0x7FC0


def poison_value(kv_dtype):
    return FP8_NAN if kv_dtype == oracle.KV_FP8 else BF16_NAN


def padded_history(inp: I.DecodeInputs, reqs=None):
    """[B][Tmax][Hkv][D] bf16 history (all tokens but this step's) and counts."""
    reqs = list(range(inp.batch.batch)) if reqs is None else list(reqs)
    w = inp.workload
    counts = np.array([inp.k_tokens[b].shape[0] - 1 for b in reqs], np.int32)
    T = max(1, int(counts.max()) if len(counts) else 1)
    k = np.zeros((len(reqs), T, w.kv_heads, w.head_dim), np.uint16)
    v = np.zeros_like(k)
    for i, b in enumerate(reqs):
        n = counts[i]
        k[i, :n] = inp.k_tokens[b][:n]
        v[i, :n] = inp.v_tokens[b][:n]
    return k, v, counts


def oracle_pool(inp: I.DecodeInputs, kv_dtype, poison=True, append=True, reqs=None):
    """Build the oracle's copy of the cache: history via the bulk writer, this
    step's token via the append (unless append=False)."""
    w = inp.workload
    fill = poison_value(kv_dtype) if poison else 0
    pool = oracle.Pool(kv_dtype, inp.num_pages, w.kv_heads, w.page_size, w.head_dim, fill=fill)
    reqs = list(range(inp.batch.batch)) if reqs is None else list(reqs)
    ks = inp.k_scale if kv_dtype == oracle.KV_FP8 else None
    vs = inp.v_scale if kv_dtype == oracle.KV_FP8 else None
    table = inp.batch.page_table[reqs]
    k, v, counts = padded_history(inp, reqs)
    oracle.kv_write(pool, table, np.zeros(len(reqs), np.int32), counts, k, v, ks, vs)
    if append:
        oracle.kv_append(pool, table, inp.batch.context_lens[reqs], inp.k_new()[reqs],
                         inp.v_new()[reqs], ks, vs)
    return pool


_E4M3 = None


def e4m3_table_torch():
    """Decode table from torch's float8_e4m3fn (independent of the oracle)."""
    global _E4M3
    if _E4M3 is None:
        _E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return _E4M3


def block_index_maps(kv_dtype, P, D):
    """Element offsets, within one head's K block and V block of a page, of
    element (slot t, dim d): the documented pool layout written out in NumPy
    (independently of the oracle's C addressing).

    Blocks are cut into segments of SEG = min(P, 64/e) tokens.
    K: a token row of D*e bytes is R = D*e/16 chunks of 16 bytes, chunk
    c = q*KL + l with KL = R/4; token u = TG*s + 4j + a of a segment (TG =
    16/e, a < 4) has chunk c at chunk position ((j*KL + l)*4 + q)*(4*NS) +
    4s + a of the segment, NS = SEG/TG.
    V: a segment is [D][SEG].
    """
    e = 1 if kv_dtype == oracle.KV_FP8 else 2
    t = np.arange(P)[:, None]
    d = np.arange(D)[None, :]
    SEG = min(P, 64 // e)
    TG, R = 16 // e, D * e // 16
    NS, KL = SEG // TG, R // 4
    seg, u = t // SEG, t % SEG
    sub, w = u // TG, u % TG
    j, a = w // 4, w % 4
    byte = d * e
    c, inner = byte // 16, byte % 16
    q, l = c // KL, c % KL
    k_bytes = seg * SEG * D * e + (((j * KL + l) * 4 + q) * (4 * NS) + 4 * sub + a) * 16 + inner
    v_off = (seg * D + d) * SEG + u
    return (k_bytes // e).astype(np.int64), v_off.astype(np.int64)


def kv_rows(pool, pages, slots):
    """K and V of (page, slot) pairs for every head: arrays [n][Hkv][D] of raw
    codes / bf16 bits, read from the pool by the documented layout."""
    kmap, vmap = block_index_maps(pool.kv_dtype, pool.P, pool.D)
    pages = np.asarray(pages, np.int64)[:, None, None]
    slots = np.asarray(slots, np.int64)
    heads = np.arange(pool.Hkv, dtype=np.int64)[None, :, None]
    block = (pages * pool.Hkv + heads) * pool.P * pool.D
    kidx = block + kmap[slots][:, None, :]
    vidx = block + vmap[slots][:, None, :]
    return pool.k.reshape(-1)[kidx], pool.v.reshape(-1)[vidx]


def dense_kv(pool, page_row, L, kv_dtype, k_scale=None, v_scale=None):
    """Gather tokens [0, L) of one request from the pool by NumPy indexing of
    the documented layout; returns fp64 K, V [L][Hkv][D]."""
    t = np.arange(L)
    pages = np.asarray(page_row)[t // pool.P]
    slots = t % pool.P
    kc, vc = kv_rows(pool, pages, slots)
    if kv_dtype == oracle.KV_FP8:
        tab = e4m3_table_torch()
        K = tab[kc] * np.asarray(k_scale, np.float64)[None, :, None]
        V = tab[vc] * np.asarray(v_scale, np.float64)[None, :, None]
    else:
        K = I.bf16_bits_to_f32(kc).astype(np.float64)
        V = I.bf16_bits_to_f32(vc).astype(np.float64)
    return K, V


def textbook_attention(q_bf16, K, V, sm_scale):
    """softmax(sm_scale * q K^T) V for all query heads of one request, fp64.
    q: [Hq][D] bf16 bits; K, V: [L][Hkv][D]."""
    q = I.bf16_bits_to_f32(q_bf16).astype(np.float64)
    Hq, D = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((Hq, D))
    lse = np.zeros(Hq)
    for h in range(Hq):
        s = sm_scale * (K[:, h // G, :] @ q[h])
        lse[h] = logsumexp(s)
        out[h] = np.exp(s - lse[h]) @ V[:, h // G, :]
    return out, lse


def allclose_report(got, ref, atol=2e-3, rtol=1e-2):
    """Element-wise |got - ref| <= atol + rtol*|ref|; returns (ok, max_abs, max_rel)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    ok = bool(np.all(err <= atol + rtol * np.abs(ref)))
    rel = err / np.maximum(np.abs(ref), 1e-30)
    return ok, float(err.max()) if err.size else 0.0, float(rel.max()) if rel.size else 0.0


# --- INT4 weights -------------------------------------------------------------------

def int4_rowmajor(q: np.ndarray) -> np.ndarray:
    """int8 q [N][K] in [-8, 7] -> bytes [N][K/2], feature k in the low nibble
    of byte k/2 when k is even."""
    u = (np.asarray(q, np.int16) & 15).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def int4_blocks(q: np.ndarray) -> np.ndarray:
    """The packed layout written out in NumPy (independently of the oracle's
    C addressing): 1024-byte blocks per (16 rows, 128 features), ordered
    [N/16][K/128]; byte 16*(16*kq + c) + 4*j + b of a block holds row c of
    the tile, features 32*j + 8*kq + 2*b and +1 of the group."""
    N, K = q.shape
    rm = int4_rowmajor(q)                                  # [N][K/2]
    # [nt][c][g][j][kq][b] bytes of the row-major array
    t = rm.reshape(N // 16, 16, K // 128, 4, 4, 4)
    # -> [nt][g][kq][c][j][b]
    return np.ascontiguousarray(t.transpose(0, 2, 4, 1, 3, 5)).reshape(-1)
