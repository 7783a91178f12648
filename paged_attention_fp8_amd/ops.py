"""Python binding of libpafp8 (include/pafp8.h): argument marshalling only.

Every function checks the torch tensors it is given (device, dtype, shape,
contiguity), passes their device pointers and the current HIP stream to the
C entry point of the same name, and raises if that call reports an error.
All computation happens in the library's HIP kernels; there is no fallback.
The library is loaded on first use and must have been built
(``python -m paged_attention_fp8_amd.build``).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PAFP8_LIB", os.path.join(_PKG, "libpafp8.so"))

KV_FP8_E4M3 = 0
KV_BF16 = 1
REQ_TAG_MISMATCH = 1
REQ_PAGE_OOB = 2
REQ_BAD_LEN = 4
ABI_VERSION = 2


class Pafp8Error(RuntimeError):
    pass


class _Cache(ctypes.Structure):
    _fields_ = [("kv_dtype", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


class _Batch(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_pages_per_req", ctypes.c_int32),
                ("page_table", ctypes.c_void_p), ("context_lens", ctypes.c_void_p),
                ("req_status", ctypes.c_void_p)]


_V, _I32, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_CP, _BP = ctypes.POINTER(_Cache), ctypes.POINTER(_Batch)

_SIGNATURES = {
    "page_tag_check": (_I32, [_BP, _I32, _V, _I32, _V, _V, _V]),
    "kv_quant_append": (_I32, [_CP, _BP, _V, _V, _V]),
    "kv_quant_append_checked": (_I32, [_CP, _BP, _V, _V, _V, _V, _V, _V]),
    "page_tag_realloc": (_I32, [_I32, _V, _V, _V, _V, _I32, _V, _V, _I32, _I32, _V]),
    "kv_quant_fill": (_I32, [_CP, _BP, _V, _V, _I32, _V, _V, _V]),
    "int4_pack_weights": (_I32, [_V, _I32, _I32, _V, _V]),
    "int4_gemv": (_I32, [_V, _I32, _V, _V, _I32, _I32, _V, _V]),
    "pafp8_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "pafp8_default_num_splits": (_I32, [_I32, _I32, _I32, _I32, _I32]),
    "pafp8_default_balanced_groups": (_I32, [_I32, _I32]),
    "paged_decode_attn_fp8": (_I32, [_CP, _BP, _V, _I32, _F, _I32, _V, _SZ, _V, _V, _V]),
    "paged_decode_attn_bf16": (_I32, [_CP, _BP, _V, _I32, _F, _I32, _V, _SZ, _V, _V, _V]),
    "paged_decode_attn_fp8_append": (_I32, [_CP, _BP, _V, _I32, _F, _I32, _V, _SZ, _V, _V, _V, _V, _V]),
    "paged_decode_attn_bf16_append": (_I32, [_CP, _BP, _V, _I32, _F, _I32, _V, _SZ, _V, _V, _V, _V, _V]),
    "paged_decode_attn_fp8_noalloc": (_I32, [_CP, _BP, _V, _I32, _F, _I32, _V, _V, _V]),
    "pafp8_noalloc_scratch_bytes": (_SZ, []),
    "splitk_combine": (_I32, [_V, _V, _I32, _I32, _I32, _I32, _V, _V, _V, _V]),
    "pafp8_stream_read": (_I32, [_V, _I64, _I32, _V, _I64, _V]),
    "pafp8_stream_read_write": (_I32, [_V, _I64, _V, _I64, _I32, _V]),
    "pafp8_e4m3_encode": (_I32, [_V, _V, _I64, _V]),
    "pafp8_e4m3_decode": (_I32, [_V, _V, _V, _V, _I64, _V]),
    "pafp8_status_string": (ctypes.c_char_p, [_I32]),
    "pafp8_last_error": (ctypes.c_char_p, []),
    "pafp8_abi_version": (_I32, [ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libpafp8.so (after torch, so that both use torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise Pafp8Error(f"{LIB_PATH} is not built; run `python -m paged_attention_fp8_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    sc, sb = _SZ(0), _SZ(0)
    ver = L.pafp8_abi_version(ctypes.byref(sc), ctypes.byref(sb))
    if ver != ABI_VERSION or sc.value != ctypes.sizeof(_Cache) or sb.value != ctypes.sizeof(_Batch):
        raise Pafp8Error(f"libpafp8 ABI mismatch: version {ver}, struct sizes {sc.value}/{sb.value}")
    _lib = L
    return L


def _check(status: int, what: str) -> None:
    if status != 0:
        L = lib()
        raise Pafp8Error(f"{what}: {L.pafp8_status_string(status).decode()}: "
                         f"{L.pafp8_last_error().decode()}")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


class PreparedCall:
    """One entry-point call with its arguments checked and marshalled once:
    run() only issues it on a stream (the current stream of the call's device
    unless a stream handle is given).  The tensors it was prepared with must
    stay alive with the same shapes; their contents may change between runs
    (a decode loop rewrites q, lengths and tables in place).  For loops
    where the per-call argument checks would cost more than the kernels."""

    def __init__(self, fn, args, what, device, keep, result):
        self._fn, self._args, self._what, self._dev = fn, tuple(args), what, device
        self._keep = keep          # ctypes structs the args point at
        self.result = result

    def run(self, stream: Optional[int] = None):
        st = _stream(self._dev) if stream is None else stream
        status = self._fn(*self._args, st)
        if status != 0:
            _check(status, self._what)
        return self.result


# ----------------------------------------------------------------------------
# the two objects of the ABI
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class PagedKVCache:
    """The shared physical page pool.  The tensors are shaped [pages][Hkv][P][D]
    (K) and [pages][Hkv][D][P] (V) as containers only: the P*D elements of a
    (page, KV head) block are ordered by the segmented block layout of
    include/pafp8.h, and only the library's calls write them."""
    k_pool: torch.Tensor           # uint8 (e4m3 codes) or bfloat16
    v_pool: torch.Tensor
    k_scale: Optional[torch.Tensor] = None   # float32 [Hkv], e4m3 only
    v_scale: Optional[torch.Tensor] = None

    @property
    def kv_dtype(self) -> int:
        return KV_BF16 if self.k_pool.dtype == torch.bfloat16 else KV_FP8_E4M3

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_pool.shape[1])

    @property
    def page_size(self) -> int:
        return int(self.k_pool.shape[2])

    @property
    def head_dim(self) -> int:
        return int(self.k_pool.shape[3])

    @property
    def device(self) -> torch.device:
        return self.k_pool.device

    @staticmethod
    def allocate(num_pages, num_kv_heads, page_size, head_dim, kv_dtype=KV_FP8_E4M3,
                 device="cuda", k_scale=None, v_scale=None) -> "PagedKVCache":
        dt = torch.uint8 if kv_dtype == KV_FP8_E4M3 else torch.bfloat16
        k = torch.empty((num_pages, num_kv_heads, page_size, head_dim), dtype=dt, device=device)
        v = torch.empty((num_pages, num_kv_heads, head_dim, page_size), dtype=dt, device=device)
        return PagedKVCache(k, v, k_scale, v_scale)

    def _struct(self) -> _Cache:
        P, Hkv, D = self.page_size, self.num_kv_heads, self.head_dim
        if self.kv_dtype == KV_FP8_E4M3:
            _need(self.k_pool, "k_pool", torch.uint8)
        else:
            _need(self.k_pool, "k_pool", torch.bfloat16)
        _need(self.v_pool, "v_pool", self.k_pool.dtype, (self.num_pages, Hkv, D, P), self.device)
        scales = (None, None)
        if self.kv_dtype == KV_FP8_E4M3:
            if self.k_scale is None or self.v_scale is None:
                raise ValueError("an e4m3 cache needs k_scale and v_scale")
            _need(self.k_scale, "k_scale", torch.float32, (Hkv,), self.device)
            _need(self.v_scale, "v_scale", torch.float32, (Hkv,), self.device)
            scales = (self.k_scale.data_ptr(), self.v_scale.data_ptr())
        return _Cache(self.kv_dtype, self.num_pages, P, Hkv, D, 0, self.k_pool.data_ptr(),
                      self.v_pool.data_ptr(), scales[0], scales[1])


@dataclasses.dataclass
class DecodeBatch:
    """One decode step's requests: page tables, lengths, and (optionally) the
    per-request verdict of page_tag_check (None = no-op tracker)."""
    page_table: torch.Tensor                 # int32 [B][max_pages]
    context_lens: torch.Tensor               # int32 [B]
    req_status: Optional[torch.Tensor] = None  # int32 [B]

    @property
    def batch(self) -> int:
        return int(self.page_table.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    def with_status(self, req_status: Optional[torch.Tensor]) -> "DecodeBatch":
        return DecodeBatch(self.page_table, self.context_lens, req_status)

    def _struct(self, device) -> _Batch:
        B = self.batch
        _need(self.page_table, "page_table", torch.int32, device=device)
        if self.page_table.dim() != 2:
            raise ValueError("page_table must be [B][max_pages]")
        _need(self.context_lens, "context_lens", torch.int32, (B,), device)
        if self.req_status is not None:
            _need(self.req_status, "req_status", torch.int32, (B,), device)
        return _Batch(B, self.max_pages, self.page_table.data_ptr(),
                      self.context_lens.data_ptr(), _ptr(self.req_status))


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------

def _tag_check_call(batch: DecodeBatch, page_size: int, page_tags: torch.Tensor,
                    expected_tags: torch.Tensor, out: Optional[torch.Tensor]) -> PreparedCall:
    dev = batch.page_table.device
    bs = batch._struct(dev)
    # tags are 32-bit patterns; int32 and uint32 tensors are both accepted
    tag_dtype = page_tags.dtype if page_tags.dtype in (torch.int32, torch.uint32) else torch.int32
    _need(page_tags, "page_tags", tag_dtype, device=dev)
    _need(expected_tags, "expected_tags", tag_dtype, tuple(batch.page_table.shape), dev)
    if out is None:
        out = torch.empty(batch.batch, dtype=torch.int32, device=dev)
    _need(out, "req_status_out", torch.int32, (batch.batch,), dev)
    return PreparedCall(lib().page_tag_check,
                        (ctypes.byref(bs), page_size, page_tags.data_ptr(), page_tags.numel(),
                         expected_tags.data_ptr(), out.data_ptr()),
                        "page_tag_check", dev, (bs, batch, page_tags, expected_tags), out)


def page_tag_check(batch: DecodeBatch, page_size: int, page_tags: torch.Tensor,
                   expected_tags: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-request status (0 = OK, else PAFP8_REQ_* flags)."""
    return _tag_check_call(batch, page_size, page_tags, expected_tags, out).run()


def prepare_page_tag_check(batch: DecodeBatch, page_size: int, page_tags: torch.Tensor,
                           expected_tags: torch.Tensor, out: torch.Tensor) -> PreparedCall:
    """page_tag_check as a PreparedCall writing `out`."""
    return _tag_check_call(batch, page_size, page_tags, expected_tags, out)


def _kv_src(t, name, shape, dev):
    _need(t, name, torch.bfloat16, shape, dev)


def kv_quant_append(cache: PagedKVCache, batch: DecodeBatch, k_new: torch.Tensor,
                    v_new: torch.Tensor) -> None:
    """Write this step's token (bf16 [B][Hkv][D]) of every request into its page."""
    dev = cache.device
    cs, bs = cache._struct(), batch._struct(dev)
    shape = (batch.batch, cache.num_kv_heads, cache.head_dim)
    _kv_src(k_new, "k_new", shape, dev)
    _kv_src(v_new, "v_new", shape, dev)
    _check(lib().kv_quant_append(ctypes.byref(cs), ctypes.byref(bs), k_new.data_ptr(),
                                 v_new.data_ptr(), _stream(dev)), "kv_quant_append")


def kv_quant_append_checked(cache: PagedKVCache, batch: DecodeBatch, page_tags: torch.Tensor,
                            expected_tags: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """page_tag_check and kv_quant_append in one launch; returns the per-request
    status (batch.req_status is ignored)."""
    dev = cache.device
    cs, bs = cache._struct(), batch._struct(dev)
    shape = (batch.batch, cache.num_kv_heads, cache.head_dim)
    _kv_src(k_new, "k_new", shape, dev)
    _kv_src(v_new, "v_new", shape, dev)
    tag_dtype = page_tags.dtype if page_tags.dtype in (torch.int32, torch.uint32) else torch.int32
    _need(page_tags, "page_tags", tag_dtype, (cache.num_pages,), dev)
    _need(expected_tags, "expected_tags", tag_dtype, tuple(batch.page_table.shape), dev)
    if out is None:
        out = torch.empty(batch.batch, dtype=torch.int32, device=dev)
    _need(out, "req_status_out", torch.int32, (batch.batch,), dev)
    _check(lib().kv_quant_append_checked(ctypes.byref(cs), ctypes.byref(bs), page_tags.data_ptr(),
                                         expected_tags.data_ptr(), k_new.data_ptr(),
                                         v_new.data_ptr(), out.data_ptr(), _stream(dev)),
           "kv_quant_append_checked")
    return out


def page_tag_realloc(page_ids: torch.Tensor, page_tags: torch.Tensor,
                     owner_req: Optional[torch.Tensor] = None,
                     owner_slot: Optional[torch.Tensor] = None,
                     page_table: Optional[torch.Tensor] = None,
                     expected_tags: Optional[torch.Tensor] = None) -> None:
    """Bump the tag of every listed page (in place) and record new owners."""
    dev = page_tags.device
    n = int(page_ids.numel())
    _need(page_ids, "page_ids", torch.int32, (n,), dev)
    tag_dtype = page_tags.dtype if page_tags.dtype in (torch.int32, torch.uint32) else torch.int32
    _need(page_tags, "page_tags", tag_dtype, device=dev)
    if (owner_req is None) != (owner_slot is None):
        raise ValueError("owner_req and owner_slot go together")
    B = maxP = 0
    if owner_req is not None:
        _need(owner_req, "owner_req", torch.int32, (n,), dev)
        _need(owner_slot, "owner_slot", torch.int32, (n,), dev)
        if expected_tags is None or expected_tags.dim() != 2:
            raise ValueError("expected_tags [B][max_pages] is needed with owners")
        _need(expected_tags, "expected_tags", tag_dtype, device=dev)
        B, maxP = (int(x) for x in expected_tags.shape)
        if page_table is not None:
            _need(page_table, "page_table", torch.int32, (B, maxP), dev)
    _check(lib().page_tag_realloc(n, page_ids.data_ptr(), _ptr(owner_req), _ptr(owner_slot),
                                  page_tags.data_ptr(), page_tags.numel(), _ptr(page_table),
                                  _ptr(expected_tags), B, maxP, _stream(dev)), "page_tag_realloc")


def kv_quant_fill(cache: PagedKVCache, batch: DecodeBatch, token_start: torch.Tensor,
                  token_count: torch.Tensor, k_src: torch.Tensor, v_src: torch.Tensor) -> None:
    """Write source token j < token_count[b] of request b (bf16 [B][T][Hkv][D])
    at position token_start[b] + j."""
    dev = cache.device
    cs, bs = cache._struct(), batch._struct(dev)
    B = batch.batch
    if k_src.dim() != 4:
        raise ValueError("k_src must be [B][T][Hkv][D]")
    T = int(k_src.shape[1])
    shape = (B, T, cache.num_kv_heads, cache.head_dim)
    _kv_src(k_src, "k_src", shape, dev)
    _kv_src(v_src, "v_src", shape, dev)
    _need(token_start, "token_start", torch.int32, (B,), dev)
    _need(token_count, "token_count", torch.int32, (B,), dev)
    _check(lib().kv_quant_fill(ctypes.byref(cs), ctypes.byref(bs), token_start.data_ptr(),
                               token_count.data_ptr(), T, k_src.data_ptr(), v_src.data_ptr(),
                               _stream(dev)), "kv_quant_fill")


def workspace_bytes(batch: int, num_q_heads: int, head_dim: int, num_splits: int) -> int:
    return int(lib().pafp8_decode_workspace_bytes(batch, num_q_heads, head_dim, num_splits))


def default_num_splits(batch: int, num_kv_heads: int, max_pages: int, page_size: int,
                       num_cus: int = 0) -> int:
    return int(lib().pafp8_default_num_splits(batch, num_kv_heads, max_pages, page_size, num_cus))


def default_balanced_groups(num_kv_heads: int, num_cus: int = 0) -> int:
    return int(lib().pafp8_default_balanced_groups(num_kv_heads, num_cus))


BALANCED = "balanced"


def _attn_call(cache: PagedKVCache, batch: DecodeBatch, q: torch.Tensor, sm_scale: float,
               num_splits, workspace: Optional[torch.Tensor], out: Optional[torch.Tensor],
               lse: Optional[torch.Tensor], return_lse: bool, k_new: Optional[torch.Tensor],
               v_new: Optional[torch.Tensor]) -> PreparedCall:
    dev = cache.device
    cs, bs = cache._struct(), batch._struct(dev)
    if q.dim() != 3:
        raise ValueError("q must be [B][Hq][D]")
    B, Hq, D = (int(x) for x in q.shape)
    _need(q, "q", torch.bfloat16, (batch.batch, Hq, cache.head_dim), dev)
    if num_splits == BALANCED:
        num_splits = -default_balanced_groups(cache.num_kv_heads)
    num_splits = int(num_splits)
    if num_splits == 0:
        num_splits = default_num_splits(B, cache.num_kv_heads, batch.max_pages, cache.page_size)
    if num_splits > 0:
        num_splits = min(num_splits, batch.max_pages)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, Hq, D), dev)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq), dev)
    need = workspace_bytes(B, Hq, D, num_splits)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace, "workspace", workspace.dtype, device=dev)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    keep = (cs, bs, cache, batch, q, workspace, k_new, v_new)
    head = (ctypes.byref(cs), ctypes.byref(bs), q.data_ptr(), Hq, float(sm_scale), num_splits,
            ws_ptr, ws_bytes)
    if k_new is not None:
        shape = (B, cache.num_kv_heads, cache.head_dim)
        _kv_src(k_new, "k_new", shape, dev)
        _kv_src(v_new, "v_new", shape, dev)
        fn = (lib().paged_decode_attn_bf16_append if cache.kv_dtype == KV_BF16
              else lib().paged_decode_attn_fp8_append)
        return PreparedCall(fn, head + (k_new.data_ptr(), v_new.data_ptr(), out.data_ptr(), _ptr(lse)),
                            "paged_decode_attn (append)", dev, keep, (out, lse))
    fn = lib().paged_decode_attn_bf16 if cache.kv_dtype == KV_BF16 else lib().paged_decode_attn_fp8
    return PreparedCall(fn, head + (out.data_ptr(), _ptr(lse)), "paged_decode_attn", dev, keep,
                        (out, lse))


def paged_decode_attn(cache: PagedKVCache, batch: DecodeBatch, q: torch.Tensor, sm_scale: float,
                      num_splits=0, workspace: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      return_lse: bool = True, k_new: Optional[torch.Tensor] = None,
                      v_new: Optional[torch.Tensor] = None):
    """Decode attention over the paged cache; dispatches to
    paged_decode_attn_fp8 or paged_decode_attn_bf16 by the pool's dtype, or,
    given this step's k_new and v_new (bf16 [B][Hkv][D]), to their _append
    forms, which write that token in the same launch.
    num_splits: S >= 1 uniform splits, 0 the library's default, -W (or
    BALANCED for pafp8_default_balanced_groups) the balanced partition over W
    work-groups per KV head.
    Returns (out fp32 [B][Hq][D], lse fp32 [B][Hq] or None)."""
    return _attn_call(cache, batch, q, sm_scale, num_splits, workspace, out, lse, return_lse,
                      k_new, v_new).run()


def prepare_paged_decode_attn(cache: PagedKVCache, batch: DecodeBatch, q: torch.Tensor,
                              sm_scale: float, num_splits=0,
                              workspace: Optional[torch.Tensor] = None,
                              out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                              return_lse: bool = True, k_new: Optional[torch.Tensor] = None,
                              v_new: Optional[torch.Tensor] = None) -> PreparedCall:
    """paged_decode_attn as a PreparedCall (same arguments); run() returns
    (out, lse).  A workspace it allocates is kept with it."""
    return _attn_call(cache, batch, q, sm_scale, num_splits, workspace, out, lse, return_lse,
                      k_new, v_new)


def paged_decode_attn_noalloc(cache: PagedKVCache, batch: DecodeBatch, q: torch.Tensor,
                              sm_scale: float, num_splits: int = 0,
                              out: Optional[torch.Tensor] = None,
                              lse: Optional[torch.Tensor] = None):
    """paged_decode_attn_fp8_noalloc: e4m3 attention with the split partials
    in the library's own device scratch (no workspace).  num_splits as for
    paged_decode_attn (BALANCED allowed); out and lse, when given, are
    written in place.  Returns (out, lse)."""
    dev = cache.device
    if cache.kv_dtype != KV_FP8_E4M3:
        raise ValueError("paged_decode_attn_noalloc needs an e4m3 pool")
    cs, bs = cache._struct(), batch._struct(dev)
    if q.dim() != 3:
        raise ValueError("q must be [B][Hq][D]")
    B, Hq, D = (int(x) for x in q.shape)
    _need(q, "q", torch.bfloat16, (batch.batch, Hq, cache.head_dim), dev)
    if num_splits == BALANCED:
        num_splits = -default_balanced_groups(cache.num_kv_heads)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, Hq, D), dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq), dev)
    _check(lib().paged_decode_attn_fp8_noalloc(ctypes.byref(cs), ctypes.byref(bs), q.data_ptr(), Hq,
                                               float(sm_scale), int(num_splits), out.data_ptr(),
                                               _ptr(lse), _stream(dev)),
           "paged_decode_attn_fp8_noalloc")
    return out, lse


def noalloc_scratch_bytes() -> int:
    return int(lib().pafp8_noalloc_scratch_bytes())


def splitk_combine(part_o: torch.Tensor, part_lse: torch.Tensor,
                   req_status: Optional[torch.Tensor] = None, out=None, lse=None):
    """Merge fp32 partials [B][Hq][S][D] / [B][Hq][S]; returns (out, lse)."""
    dev = part_o.device
    if part_o.dim() != 4:
        raise ValueError("part_o must be [B][Hq][S][D]")
    B, Hq, S, D = (int(x) for x in part_o.shape)
    _need(part_o, "part_o", torch.float32, device=dev)
    _need(part_lse, "part_lse", torch.float32, (B, Hq, S), dev)
    if req_status is not None:
        _need(req_status, "req_status", torch.int32, (B,), dev)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, Hq, D), dev)
    _need(lse, "lse", torch.float32, (B, Hq), dev)
    _check(lib().splitk_combine(part_o.data_ptr(), part_lse.data_ptr(), B, Hq, S, D,
                                _ptr(req_status), out.data_ptr(), lse.data_ptr(), _stream(dev)),
           "splitk_combine")
    return out, lse


STREAM_READ_TILE = 16384
STREAM_READ_THREADS = 256


def stream_read(buf: torch.Tensor, work_groups: int = 256,
                sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Measurement aid: one bare non-temporal read of all of buf's bytes
    (a multiple of 16 KiB) by work_groups work-groups; returns the sink of
    per-thread XORs (int32 [work_groups * 256]), whose XOR is buf's."""
    if buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty(work_groups * STREAM_READ_THREADS, dtype=torch.int32, device=buf.device)
    _need(sink, "sink", torch.int32, None, buf.device)
    _check(lib().pafp8_stream_read(buf.data_ptr(), nbytes, work_groups, sink.data_ptr(),
                                   sink.numel(), _stream(buf.device)), "pafp8_stream_read")
    return sink


def stream_read_write(src: torch.Tensor, dst: torch.Tensor, work_groups: int = 256) -> torch.Tensor:
    """Measurement aid: one bare read of all of src's bytes (a multiple of
    16 KiB) and a write of all of dst's (1/1, 1/2 or 1/4 of src's) by
    work_groups work-groups; returns dst."""
    for t, n in ((src, "src"), (dst, "dst")):
        if t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous device tensor")
    _check(lib().pafp8_stream_read_write(src.data_ptr(), src.numel() * src.element_size(), dst.data_ptr(),
                                         dst.numel() * dst.element_size(), work_groups,
                                         _stream(src.device)), "pafp8_stream_read_write")
    return dst


def e4m3_encode(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Device codec: fp32 -> e4m3 codes (uint8)."""
    _need(x, "x", torch.float32)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _need(out, "codes", torch.uint8, tuple(x.shape), x.device)
    _check(lib().pafp8_e4m3_encode(x.data_ptr(), out.data_ptr(), x.numel(), _stream(x.device)),
           "pafp8_e4m3_encode")
    return out


def e4m3_decode(codes: torch.Tensor):
    """Device codec: codes -> (fp32 direct, via fp16, via bf16), each widened to fp32."""
    _need(codes, "codes", torch.uint8)
    outs = [torch.empty(codes.shape, dtype=torch.float32, device=codes.device) for _ in range(3)]
    _check(lib().pafp8_e4m3_decode(codes.data_ptr(), outs[0].data_ptr(), outs[1].data_ptr(),
                                   outs[2].data_ptr(), codes.numel(), _stream(codes.device)),
           "pafp8_e4m3_decode")
    return tuple(outs)


# ----------------------------------------------------------------------------
# INT4 weight streaming
# ----------------------------------------------------------------------------

def int4_pack_weights(w_rowmajor: torch.Tensor, N: int, K: int,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Row-major int4 weights (uint8 [N][K/2], low nibble = even feature) to
    the packed layout int4_gemv reads (uint8 [N*K/2])."""
    dev = w_rowmajor.device
    _need(w_rowmajor, "w_rowmajor", torch.uint8, (N, K // 2), dev)
    if out is None:
        out = torch.empty(N * K // 2, dtype=torch.uint8, device=dev)
    _need(out, "w_packed", torch.uint8, (N * K // 2,), dev)
    _check(lib().int4_pack_weights(w_rowmajor.data_ptr(), N, K, out.data_ptr(), _stream(dev)),
           "int4_pack_weights")
    return out


def int4_gemv(x: torch.Tensor, w_packed: torch.Tensor, scales: torch.Tensor, N: int, K: int,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[M][N] = x[M][K] . (q * scale)^T with packed int4 weights and bf16
    scales [K/128][N]; fp32 output."""
    dev = x.device
    if x.dim() != 2:
        raise ValueError("x must be [M][K]")
    M = int(x.shape[0])
    _need(x, "x", torch.bfloat16, (M, K), dev)
    _need(w_packed, "w_packed", torch.uint8, (N * K // 2,), dev)
    _need(scales, "scales", torch.bfloat16, (K // 128, N), dev)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=dev)
    _need(out, "y", torch.float32, (M, N), dev)
    _check(lib().int4_gemv(x.data_ptr(), M, w_packed.data_ptr(), scales.data_ptr(), N, K,
                           out.data_ptr(), _stream(dev)), "int4_gemv")
    return out

