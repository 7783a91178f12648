"""The C-ABI library loads, exports every function include/pafp8.h declares,
and its host-side logic (sizing, split choice, argument validation) works
without a GPU: validation runs before any HIP call."""
import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (loads torch's HIP runtime first, as the binding does)

from paged_attention_fp8_amd import build as B
from paged_attention_fp8_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pafp8.h")


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?(?:pafp8_status|size_t|int32_t|char)\s*\*?\s*(\w+)\s*\(",
                      text, flags=re.M)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB):
        B.build()
    return ops.lib()


def test_header_declares_the_path():
    names = set(declared_functions())
    for n in ["page_tag_check", "kv_quant_append", "kv_quant_fill", "kv_quant_append_checked",
              "page_tag_realloc", "int4_pack_weights", "int4_gemv", "paged_decode_attn_fp8",
              "paged_decode_attn_bf16", "splitk_combine", "pafp8_decode_workspace_bytes",
              "pafp8_default_num_splits", "pafp8_status_string", "pafp8_last_error",
              "pafp8_abi_version", "pafp8_e4m3_encode", "pafp8_e4m3_decode"]:
        assert n in names, n


def test_every_declared_symbol_is_exported(L):
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing
    # and the binding wraps each of them
    assert set(declared_functions()) <= set(ops._SIGNATURES)


def test_single_hip_runtime_mapped(L):
    with open("/proc/self/maps") as f:
        maps = f.read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(paths) == 1, paths


def test_abi_version_and_struct_sizes(L):
    sc, sb = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.pafp8_abi_version(ctypes.byref(sc), ctypes.byref(sb)) == ops.ABI_VERSION
    assert sc.value == ctypes.sizeof(ops._Cache) == 56
    assert sb.value == ctypes.sizeof(ops._Batch) == 32


def test_status_strings(L):
    assert L.pafp8_status_string(0) == b"PAFP8_OK"
    assert L.pafp8_status_string(1) == b"PAFP8_EINVAL"
    assert L.pafp8_status_string(2) == b"PAFP8_EUNSUPPORTED"
    assert L.pafp8_status_string(3) == b"PAFP8_EHIP"
    assert L.pafp8_status_string(77) == b"PAFP8_UNKNOWN"


def test_workspace_bytes(L):
    assert L.pafp8_decode_workspace_bytes(64, 64, 128, 1) == 0
    assert L.pafp8_decode_workspace_bytes(64, 64, 128, 2) == 64 * 64 * 2 * (128 + 1) * 4
    assert L.pafp8_decode_workspace_bytes(0, 64, 128, 8) == 0


def test_default_split_choice(L):
    # about one work-group per CU
    assert L.pafp8_default_num_splits(64, 8, 256, 64, 256) == 1
    assert L.pafp8_default_num_splits(32, 8, 256, 64, 256) == 1
    assert L.pafp8_default_num_splits(16, 8, 256, 64, 256) == 2
    assert L.pafp8_default_num_splits(8, 8, 256, 64, 256) == 4
    assert L.pafp8_default_num_splits(4, 8, 4096, 64, 256) == 8
    # no split shorter than 512 tokens, and none below 2048 tokens
    assert L.pafp8_default_num_splits(1, 8, 256, 64, 256) == 32
    assert L.pafp8_default_num_splits(1, 8, 64, 64, 256) == 8
    assert L.pafp8_default_num_splits(1, 8, 32, 64, 256) == 4
    assert L.pafp8_default_num_splits(1, 4, 16, 16, 256) == 1
    assert L.pafp8_default_num_splits(2, 8, 64, 16, 256) == 1       # 1024 tokens: whole
    assert L.pafp8_default_num_splits(1, 8, 31, 64, 256) == 1       # 1984 tokens: whole
    assert L.pafp8_default_num_splits(2, 8, 128, 16, 256) == 4      # 2048 tokens: 512 each


def _cache(**kw):
    c = ops._Cache(0, 16, 64, 8, 128, 0, 256, 256 + 4096, 64, 128)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _batch(**kw):
    b = ops._Batch(4, 16, 1024, 2048, None)
    for k, v in kw.items():
        setattr(b, k, v)
    return b


def _attn(L, cache, batch, hq=64, sm=0.1, splits=1, q=4096, out=8192, fn="paged_decode_attn_fp8"):
    return getattr(L, fn)(ctypes.byref(cache) if cache is not None else None,
                          ctypes.byref(batch) if batch is not None else None,
                          q, hq, sm, splits, None, 0, out, None, None)


@pytest.mark.parametrize("case,status,msg", [
    (dict(cache=None), 1, "cache descriptor is NULL"),
    (dict(batch=None), 1, "batch descriptor is NULL"),
    (dict(cache_kw=dict(kv_dtype=1)), 1, "does not match"),
    (dict(cache_kw=dict(page_size=48)), 2, "page_size"),
    (dict(cache_kw=dict(head_dim=96)), 2, "head_dim"),
    (dict(cache_kw=dict(k_scale=None)), 1, "k_scale"),
    (dict(cache_kw=dict(k_pool=257)), 1, "aligned"),
    (dict(batch_kw=dict(max_pages_per_req=0)), 1, "max_pages_per_req"),
    (dict(batch_kw=dict(page_table=None)), 1, "page_table"),
    (dict(hq=60), 1, "multiple of num_kv_heads"),
    (dict(hq=8 * 17), 2, "group size"),
    (dict(sm=0.0), 1, "sm_scale"),
    (dict(sm=float("nan")), 1, "sm_scale"),
    (dict(splits=-1), 1, "num_splits = -1 needs a workspace"),     # balanced, W = 1
    (dict(splits=-65537), 1, "at most 65536"),
    (dict(splits=-65536, batch_kw=dict(batch=2147483000)), 2, "too large"),
    (dict(splits=4), 1, "workspace"),
    (dict(q=0), 1, "q or out is NULL"),
])
def test_attention_validation_without_gpu(L, case, status, msg):
    cache = None if case.get("cache", 1) is None else _cache(**case.get("cache_kw", {}))
    batch = None if case.get("batch", 1) is None else _batch(**case.get("batch_kw", {}))
    st = _attn(L, cache, batch, hq=case.get("hq", 64), sm=case.get("sm", 0.1),
               splits=case.get("splits", 1), q=case.get("q", 4096))
    assert msg in L.pafp8_last_error().decode(), L.pafp8_last_error()
    assert st == status
    assert msg in L.pafp8_last_error().decode()


def test_bf16_entry_rejects_fp8_pool(L):
    assert _attn(L, _cache(), _batch(), fn="paged_decode_attn_bf16") == 1
    assert b"does not match" in L.pafp8_last_error()


def test_other_entry_points_validate_without_gpu(L):
    c, b = _cache(), _batch()
    assert L.kv_quant_append(ctypes.byref(c), ctypes.byref(b), None, 64, None) == 1
    assert L.kv_quant_fill(ctypes.byref(c), ctypes.byref(b), None, 64, 8, 64, 64, None) == 1
    assert L.kv_quant_fill(ctypes.byref(c), ctypes.byref(b), 64, 64, 0, 64, 64, None) == 1
    wide = _cache(num_kv_heads=1 << 19)     # 2^19 heads x 128 dims: 16 source rows exceed 1 GiB
    assert L.kv_quant_fill(ctypes.byref(wide), ctypes.byref(b), 64, 64, 8, 64, 64, None) == 2
    assert b"2^25" in L.pafp8_last_error()
    assert L.page_tag_check(ctypes.byref(_batch(batch=-1)), 64, 64, 10, 64, 64, None) == 1
    assert L.page_tag_check(ctypes.byref(b), 24, 64, 10, 64, 64, None) == 2
    assert L.page_tag_check(ctypes.byref(b), 64, 64, 10, None, 64, None) == 1
    assert L.splitk_combine(64, 64, 1, 8, 2, 6, None, 64, None, None) == 2
    assert L.splitk_combine(None, 64, 1, 8, 2, 128, None, 64, None, None) == 1
    assert L.kv_quant_append_checked(ctypes.byref(c), ctypes.byref(b), None, 64, 64, 64, 64, None) == 1
    assert b"page_tags" in L.pafp8_last_error()
    assert L.kv_quant_append_checked(ctypes.byref(c), ctypes.byref(b), 64, 64, 64, 64, None, None) == 1
    assert L.page_tag_realloc(-1, 64, None, None, 64, 10, None, None, 0, 0, None) == 1
    assert L.page_tag_realloc(4, None, None, None, 64, 10, None, None, 0, 0, None) == 1
    assert L.page_tag_realloc(4, 64, 64, None, 64, 10, None, 64, 4, 16, None) == 1
    assert b"both" in L.pafp8_last_error()
    assert L.page_tag_realloc(4, 64, 64, 64, 64, 10, None, None, 4, 16, None) == 1
    assert b"expected_tags" in L.pafp8_last_error()
    assert L.page_tag_realloc(0, None, None, None, None, 0, None, None, 0, 0, None) == 0
    # INT4 weight streaming: shapes, NULLs, alignment
    assert L.int4_gemv(64, 1, 64, 64, 24, 512, 64, None) == 2           # N % 16
    assert L.int4_gemv(64, 1, 64, 64, 16, 384, 64, None) == 2           # K % 512
    assert L.int4_gemv(None, 1, 64, 64, 16, 512, 64, None) == 1
    assert L.int4_gemv(72, 1, 64, 64, 16, 512, 64, None) == 1           # x not 16-byte aligned
    assert L.int4_gemv(None, 0, None, None, 16, 512, None, None) == 0   # M = 0: nothing to do
    assert L.int4_pack_weights(64, 16, 500, 64, None) == 2
    assert L.int4_pack_weights(None, 16, 512, 64, None) == 1
    assert L.int4_pack_weights(66, 16, 512, 64, None) == 1              # source not 4-byte aligned
    assert L.pafp8_e4m3_encode(None, None, -1, None) == 1
    # the bare read (a measurement aid): size, sink, pointers, alignment
    assert L.pafp8_stream_read(64, 16384 + 16, 1, 64, 256, None) == 1   # not whole 16 KiB tiles
    assert L.pafp8_stream_read(64, -16384, 1, 64, 256, None) == 1
    assert L.pafp8_stream_read(64, 16384, 0, 64, 256, None) == 1        # no work-groups
    assert L.pafp8_stream_read(64, 16384, 2, 64, 511, None) == 1        # sink one word short
    assert b"512" in L.pafp8_last_error()
    assert L.pafp8_stream_read(None, 16384, 1, 64, 256, None) == 1
    assert L.pafp8_stream_read(64, 16384, 1, None, 256, None) == 1
    assert L.pafp8_stream_read(72, 16384, 1, 64, 256, None) == 1        # src not 16-byte aligned
    assert L.pafp8_stream_read_write(64, 16384, 64, 16384 // 3, 1, None) == 1   # ratio not 1, 2, 4
    assert L.pafp8_stream_read_write(64, 16384, 64, 16384 // 8, 1, None) == 1
    assert L.pafp8_stream_read_write(64, 16384 + 16, 64, 8200, 1, None) == 1
    assert L.pafp8_stream_read_write(64, 16384, 64, 0, 1, None) == 1
    assert L.pafp8_stream_read_write(64, 0, 64, 16, 1, None) == 1
    assert L.pafp8_stream_read_write(64, 16384, 64, 8192, 0, None) == 1
    assert L.pafp8_stream_read_write(64, 16384, None, 8192, 1, None) == 1
    assert L.pafp8_stream_read_write(64, 16384, 72, 8192, 1, None) == 1       # dst not 16-byte aligned
    assert L.pafp8_stream_read_write(None, 0, None, 0, 1, None) == 0           # nothing to do
    # empty work is OK and launches nothing
    assert L.pafp8_e4m3_encode(None, None, 0, None) == 0
    assert _attn(L, _cache(), _batch(batch=0)) == 0
    assert L.page_tag_check(ctypes.byref(_batch(batch=0)), 64, None, 0, None, None, None) == 0


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(ops, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(ops, "_lib", None)
    with pytest.raises(ops.Pafp8Error, match="not built"):
        ops.lib()


def test_fused_append_entries_validate_without_gpu(L):
    """The append-in-attention entries check what the attention entries check,
    plus the new token's pointers, before any HIP call."""
    def call(fn, cache, k_new=8192, v_new=8192, batch=None):
        b = batch if batch is not None else _batch()
        return getattr(L, fn)(ctypes.byref(cache), ctypes.byref(b), 4096, 64, 0.1, 1, None, 0,
                              k_new, v_new, 8192, None, None)
    assert call("paged_decode_attn_fp8_append", _cache(), k_new=None) == 1
    assert "k_new or v_new is NULL" in L.pafp8_last_error().decode()
    assert call("paged_decode_attn_fp8_append", _cache(), v_new=None) == 1
    assert call("paged_decode_attn_bf16_append", _cache()) == 1        # e4m3 pool
    assert "does not match" in L.pafp8_last_error().decode()
    assert call("paged_decode_attn_fp8_append", _cache(), k_new=None, batch=_batch(batch=0)) == 0


def _noalloc(L, cache, batch, hq=64, splits=1):
    return L.paged_decode_attn_fp8_noalloc(ctypes.byref(cache), ctypes.byref(batch), 4096, hq, 0.1,
                                           splits, 8192, None, None)


def test_noalloc_entry_validates_without_gpu(L):
    """The no-allocation entry point checks its arguments like the workspace
    call, and refuses, before any HIP call, a split count whose partials
    exceed its fixed scratch."""
    assert L.pafp8_noalloc_scratch_bytes() == 16 << 20
    assert _noalloc(L, _cache(kv_dtype=1), _batch()) == 1
    assert b"does not match" in L.pafp8_last_error()
    assert _noalloc(L, _cache(), _batch(), hq=60) == 1
    big = _batch(batch=64)                                  # 64 x 64 heads x 16 splits x 129 floats
    assert L.pafp8_decode_workspace_bytes(64, 64, 128, 16) > 16 << 20
    assert _noalloc(L, _cache(), big, splits=16) == 2
    assert b"scratch" in L.pafp8_last_error()
    assert _noalloc(L, _cache(), _batch(batch=0), splits=16) == 0   # nothing to do
