"""CPU oracle for FP8 (e4m3) paged decode attention -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct implementation (``pafp8_oracle.c``, fp64
arithmetic from exactly decoded inputs) used by ``tests/``, by the smoke check
and by the CPU-baseline leg of ``bench.py``.  It shares no code with the HIP
library and no product code path may import it.

Each function names the passage of the pages it follows; the C file's header
lists the sources and the readings taken where the pages are silent:

* Cloudflare, "Smaller, faster, safer: running Kimi and GLM at scale"
  (translation at reed-read.pages.dev/article/2383), section "KV 缓存量化"
  (KV cache quantization) -- FP8 e4m3 storage, conversion on read;
* same post, section "共享 KV 缓存保护" (shared KV cache protection) -- per-page
  tags, per-request expected tags, check before decode reads, abort on mismatch;
* same post, section "模型权重压缩" (model weight compression) -- INT4 weights
  streamed and expanded on read during decode;
* remio.ai analysis of the post, section on shared KV cache safety -- paged
  attention maps each logical sequence onto physical pages.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against something other than itself (torch's independent float8_e4m3fn
codec, brute-force search, NumPy textbook attention on gathered pages, closed
forms, invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pafp8_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

REQ_TAG_MISMATCH = 1
REQ_PAGE_OOB = 2
REQ_BAD_LEN = 4

KV_FP8 = 0
KV_BF16 = 1

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_D = ctypes.c_double
_F = ctypes.c_float


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FMA contraction).
    src/out: another source and library path (the pins' mutation check
    compiles altered copies this way)."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_lib = None


def lib() -> ctypes.CDLL:
    """The compiled oracle; PAFP8_ORACLE_LIB names another build of it (used
    only by the pins' mutation check)."""
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(os.environ.get("PAFP8_ORACLE_LIB") or build())
        L = _lib
        L.oracle_e4m3_decode.restype = _D
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [_F]
        L.oracle_e4m3_encode_brute.restype = ctypes.c_uint8
        L.oracle_e4m3_encode_brute.argtypes = [_F]
        L.oracle_e4m3_encode_array.argtypes = [_P, _P, _I64]
        L.oracle_e4m3_encode_brute_array.argtypes = [_P, _P, _I64]
        L.oracle_e4m3_encode_bits_range.argtypes = [ctypes.c_uint32, _I64, _P]
        L.oracle_quantize.restype = ctypes.c_uint8
        L.oracle_quantize.argtypes = [ctypes.c_uint16, _F]
        L.oracle_k_offset.restype = _I64
        L.oracle_k_offset.argtypes = [_I, _I64, _I, _I, _I, _I, _I, _I]
        L.oracle_v_offset.restype = _I64
        L.oracle_v_offset.argtypes = [_I, _I64, _I, _I, _I, _I, _I, _I]
        L.oracle_kv_write.argtypes = [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _I, _P,
                                      _P, _P, _P, _P, _P, _P]
        L.oracle_kv_append.argtypes = [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P,
                                       _P, _P, _P, _P, _P, _P]
        L.oracle_page_tag_check.argtypes = [_I, _I, _I, _P, _P, _P, _P, _I, _P]
        L.oracle_page_tag_realloc.argtypes = [_I, _P, _P, _P, _P, _I, _P, _P, _I, _I]
        L.oracle_int4_unpack.argtypes = [_P, _I, _I, _P]
        L.oracle_int4_gemv.argtypes = [_I, _I, _I, _P, _P, _P, _P]
        L.oracle_paged_attention.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P,
                                             _P, _P, _P, _P, _P, _D, _P, _P]
        L.oracle_attention_range.argtypes = [_I, _I, _I, _I, _I, _I, _I, _P, _I, _I,
                                             _P, _P, _P, _P, _P, _D, _I64, _I64, _P, _P]
        L.oracle_splitk_combine.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P]
        L.oracle_num_threads.restype = _I
    return _lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# --- O1 / O2: the e4m3 codec -------------------------------------------------

def e4m3_decode(code: int) -> float:
    """Value of one e4m3 code (OCP E4M3 reading of the pages' "FP8 (e4m3)")."""
    return lib().oracle_e4m3_decode(int(code) & 0xFF)


def e4m3_decode_table() -> np.ndarray:
    """fp64 values of all 256 codes (NaN for 0x7F and 0xFF)."""
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(x) -> np.ndarray:
    """Round-to-nearest-even, saturating encoder (arithmetic form), elementwise."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32).reshape(-1))
    out = np.empty(x.shape, np.uint8)
    lib().oracle_e4m3_encode_array(_ptr(x), _ptr(out), x.size)
    return out


def e4m3_encode_brute(x) -> np.ndarray:
    """The encoder's definition: nearest finite code by exhaustive search."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32).reshape(-1))
    out = np.empty(x.shape, np.uint8)
    lib().oracle_e4m3_encode_brute_array(_ptr(x), _ptr(out), x.size)
    return out


def e4m3_encode_bits_range(first: int, n: int) -> np.ndarray:
    """Codes of the fp32 values with bit patterns first .. first+n-1."""
    out = np.empty(n, np.uint8)
    lib().oracle_e4m3_encode_bits_range(ctypes.c_uint32(first), n, _ptr(out))
    return out


def quantize(x_bf16: int, scale: float) -> int:
    """enc(f32(x) / scale) with an IEEE single division."""
    return lib().oracle_quantize(int(x_bf16) & 0xFFFF, float(np.float32(scale)))


# --- O5: pool writes ----------------------------------------------------------

class Pool:
    """Host copy of the physical page pool in the documented layout.

    Arrays of shape [num_pages][Hkv][P][D] (K) and [num_pages][Hkv][D][P]
    (V), the device tensors' shapes; the last two axes hold one head's block
    of a page in the element order the library documents (see k_offset /
    v_offset), which is not [slot][dim] / [dim][slot] in general.
    uint8 e4m3 codes (kv_dtype 0) or uint16 bf16 bit patterns (kv_dtype 1).
    """

    def __init__(self, kv_dtype, num_pages, Hkv, P, D, fill=0):
        e = 1 if kv_dtype == KV_FP8 else 2
        if (D * e) % 64 or P % (16 // e) or P & (P - 1):
            raise ValueError(f"the pool layout needs head_dim*e % 64 == 0 and a power-of-two page "
                             f"of at least {16 // e} tokens (got D={D}, P={P})")
        self.kv_dtype, self.num_pages, self.Hkv, self.P, self.D = kv_dtype, num_pages, Hkv, P, D
        dt = np.uint8 if kv_dtype == KV_FP8 else np.uint16
        self.k = np.full((num_pages, Hkv, P, D), fill, dtype=dt)
        self.v = np.full((num_pages, Hkv, D, P), fill, dtype=dt)


def kv_write(pool: Pool, page_table, start, count, k_src, v_src, k_scale=None, v_scale=None,
             status=None):
    """Write request b's source tokens j < count[b] at positions start[b] + j."""
    page_table = _c(page_table, np.int32)
    B, maxP = page_table.shape
    start, count = _c(start, np.int32), _c(count, np.int32)
    k_src, v_src = _c(k_src, np.uint16), _c(v_src, np.uint16)
    T_src = k_src.shape[1]
    lib().oracle_kv_write(pool.kv_dtype, B, maxP, pool.P, pool.Hkv, pool.D, pool.num_pages,
                          _ptr(page_table), _ptr(start), _ptr(count), T_src,
                          _ptr(_c(status, np.int32)), _ptr(k_src), _ptr(v_src),
                          _ptr(_c(k_scale, np.float32)), _ptr(_c(v_scale, np.float32)),
                          _ptr(pool.k), _ptr(pool.v))


def kv_append(pool: Pool, page_table, context_lens, k_new, v_new, k_scale=None, v_scale=None,
              status=None):
    """Decode-step append of one token per request at position context_lens[b] - 1."""
    page_table = _c(page_table, np.int32)
    B, maxP = page_table.shape
    lib().oracle_kv_append(pool.kv_dtype, B, maxP, pool.P, pool.Hkv, pool.D, pool.num_pages,
                           _ptr(page_table), _ptr(_c(context_lens, np.int32)),
                           _ptr(_c(status, np.int32)), _ptr(_c(k_new, np.uint16)),
                           _ptr(_c(v_new, np.uint16)), _ptr(_c(k_scale, np.float32)),
                           _ptr(_c(v_scale, np.float32)), _ptr(pool.k), _ptr(pool.v))


def k_offset(kv_dtype, page, g, slot, d, Hkv, P, D) -> int:
    """Element offset of K (page, head g, slot, dim d) in the pool."""
    return lib().oracle_k_offset(kv_dtype, page, g, slot, d, Hkv, P, D)


def v_offset(kv_dtype, page, g, slot, d, Hkv, P, D) -> int:
    """Element offset of V (page, head g, slot, dim d) in the pool."""
    return lib().oracle_v_offset(kv_dtype, page, g, slot, d, Hkv, P, D)


# --- O6: tag check --------------------------------------------------------------

def page_tag_check(page_table, context_lens, expected_tags, page_tags, page_size) -> np.ndarray:
    page_table = _c(page_table, np.int32)
    B, maxP = page_table.shape
    page_tags = _c(page_tags, np.uint32)
    out = np.empty(B, np.int32)
    lib().oracle_page_tag_check(B, maxP, page_size, _ptr(page_table),
                                _ptr(_c(context_lens, np.int32)),
                                _ptr(_c(expected_tags, np.uint32)), _ptr(page_tags),
                                page_tags.size, _ptr(out))
    return out


def page_tag_realloc(page_ids, page_tags, owner_req=None, owner_slot=None, page_table=None,
                     expected_tags=None):
    """Reallocation in list order; returns updated copies (page_tags,
    page_table or None, expected_tags or None)."""
    ids = _c(page_ids, np.int32)
    tags = np.array(page_tags, np.uint32, copy=True)
    table = None if page_table is None else np.array(page_table, np.int32, copy=True)
    exp = None if expected_tags is None else np.array(expected_tags, np.uint32, copy=True)
    shape = table.shape if table is not None else (exp.shape if exp is not None else (0, 0))
    B, maxP = shape
    req = None if owner_req is None else _c(owner_req, np.int32)
    slot = None if owner_slot is None else _c(owner_slot, np.int32)
    lib().oracle_page_tag_realloc(ids.size, _ptr(ids), _ptr(req), _ptr(slot), _ptr(tags), tags.size,
                                  _ptr(table), _ptr(exp), B, maxP)
    return tags, table, exp


# --- O7 / O8: attention and combine ---------------------------------------------

def paged_attention(pool: Pool, q_bf16, page_table, context_lens, sm_scale, k_scale=None,
                    v_scale=None, status=None):
    """fp64 decode attention; returns (out [B][Hq][D] fp64, lse [B][Hq] fp64)."""
    q = _c(q_bf16, np.uint16)
    B, Hq, D = q.shape
    page_table = _c(page_table, np.int32)
    maxP = page_table.shape[1]
    out = np.empty((B, Hq, D), np.float64)
    lse = np.empty((B, Hq), np.float64)
    lib().oracle_paged_attention(pool.kv_dtype, B, Hq, pool.Hkv, D, pool.P, maxP, pool.num_pages,
                                 _ptr(page_table), _ptr(_c(context_lens, np.int32)),
                                 _ptr(_c(status, np.int32)), _ptr(q), _ptr(pool.k), _ptr(pool.v),
                                 _ptr(_c(k_scale, np.float32)), _ptr(_c(v_scale, np.float32)),
                                 float(sm_scale), _ptr(out), _ptr(lse))
    return out, lse


def attention_range(pool: Pool, q_bf16, page_table, b, h, t0, t1, sm_scale, k_scale=None,
                    v_scale=None):
    """Partial (o [D], lse) of request b, query head h over tokens [t0, t1)."""
    q = _c(q_bf16, np.uint16)
    B, Hq, D = q.shape
    page_table = _c(page_table, np.int32)
    o = np.empty(D, np.float64)
    lse = np.empty(1, np.float64)
    lib().oracle_attention_range(pool.kv_dtype, Hq, pool.Hkv, D, pool.P, page_table.shape[1],
                                 pool.num_pages, _ptr(page_table), b, h, _ptr(q), _ptr(pool.k),
                                 _ptr(pool.v), _ptr(_c(k_scale, np.float32)),
                                 _ptr(_c(v_scale, np.float32)), float(sm_scale), t0, t1,
                                 _ptr(o), _ptr(lse))
    return o, float(lse[0])


def splitk_combine(part_o, part_lse, status=None):
    """fp64 log-sum-exp combine of fp32 partials [B][Hq][S][D] and [B][Hq][S]."""
    part_o = _c(part_o, np.float32)
    part_lse = _c(part_lse, np.float32)
    B, Hq, S, D = part_o.shape
    out = np.empty((B, Hq, D), np.float64)
    lse = np.empty((B, Hq), np.float64)
    lib().oracle_splitk_combine(B, Hq, S, D, _ptr(part_o), _ptr(part_lse),
                                _ptr(_c(status, np.int32)), _ptr(out), _ptr(lse))
    return out, lse


def num_threads() -> int:
    return lib().oracle_num_threads()


# --- INT4 weight streaming --------------------------------------------------------

def int4_unpack(w_packed, N, K) -> np.ndarray:
    """q [N][K] int8 from the packed layout (the oracle's own addressing)."""
    w = _c(w_packed, np.uint8)
    q = np.empty((N, K), np.int8)
    lib().oracle_int4_unpack(_ptr(w), N, K, _ptr(q))
    return q


def int4_gemv(x_bf16, w_packed, scales_bf16, N, K) -> np.ndarray:
    """y[m][n] = sum_k x[m][k] q[n][k] s[k/128][n] in fp64; x [M][K] and
    scales [K/128][N] as bf16 bit patterns."""
    x = _c(x_bf16, np.uint16)
    M = x.shape[0]
    y = np.empty((M, N), np.float64)
    lib().oracle_int4_gemv(M, N, K, _ptr(x), _ptr(_c(w_packed, np.uint8)),
                           _ptr(_c(scales_bf16, np.uint16)), _ptr(y))
    return y

