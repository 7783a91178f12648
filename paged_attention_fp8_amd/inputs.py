"""Seeded synthetic inputs for decode attention over a paged KV cache.

This module is the one place both sides draw their inputs from: the tests feed
its arrays to the CPU oracle and to the HIP library alike.  It holds none of
the method's arithmetic -- no e4m3 encoding, no attention, no tag comparison --
only the input recipe:

* bf16 tensors drawn from N(0, 1) (fp32 draws rounded to bf16, nearest-even),
  optionally with a fraction of elements multiplied by an outlier factor;
* per-KV-head FP8 scales amax / 448, where amax is taken over the bulk of the
  data (before outliers are injected, so that outliers do saturate);
* a host-side physical page pool: a free list in shuffled (fragmented) order
  and a per-page generation tag that is bumped on every allocation, as the
  shared-cache protection section of Cloudflare's "Smaller, faster, safer:
  running Kimi and GLM at scale" describes (section "共享 KV 缓存保护",
  shared KV cache protection: tags change whenever a page is reallocated and
  the server records the pages and tags each request expects);
* per-request page tables, expected tags and context lengths, plus injection
  of stale tags (a page freed and handed to another owner).

The named workloads mirror the shapes, length mixes and value distributions of
the decode workloads this library is measured on; each is named by what it is.
"""
from __future__ import annotations

import collections
import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

FP8_MAX = 448.0  # largest finite e4m3 magnitude; the scale maps amax onto it


# ----------------------------------------------------------------------------
# seeded generators
# ----------------------------------------------------------------------------

def rng(seed: int, *stream: int) -> np.random.Generator:
    """Independent PCG64 stream for (seed, stream...)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, stream)])))


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return rounded


def bf16_bits_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def normal_bf16(g: np.random.Generator, shape, outlier_frac: float = 0.0,
                outlier_mult: float = 20.0):
    """N(0,1) bf16 bits, with a Bernoulli(outlier_frac) subset multiplied by
    outlier_mult.  Returns (bits, bulk_amax) where bulk_amax is the largest
    magnitude before outliers were injected."""
    x = g.standard_normal(shape, dtype=np.float32)
    bulk = f32_to_bf16_bits(x)
    bulk_amax = float(np.max(np.abs(bf16_bits_to_f32(bulk)))) if bulk.size else 0.0
    if outlier_frac > 0.0:
        mask = g.random(shape, dtype=np.float32) < outlier_frac
        x = np.where(mask, x * np.float32(outlier_mult), x)
        return f32_to_bf16_bits(x), bulk_amax
    return bulk, bulk_amax


def fp8_scale_from_amax(amax) -> np.ndarray:
    """Per-head dequantisation scale amax / 448 in fp32 (1.0 where amax is 0)."""
    a = np.asarray(amax, dtype=np.float32)
    s = a / np.float32(FP8_MAX)
    return np.where(a > 0, s, np.float32(1.0)).astype(np.float32)


# ----------------------------------------------------------------------------
# host page pool with generation tags
# ----------------------------------------------------------------------------

class PoolExhausted(RuntimeError):
    """No free physical page is left for an allocation."""


class PagePool:
    """Free list over num_pages physical pages plus a uint32 tag per page.

    Every allocation bumps the page's tag (a generation counter), so a request
    that recorded an earlier tag for a page can tell that the page has since
    been handed to someone else.
    """

    def __init__(self, num_pages: int, seed: int = 0, order: str = "shuffled", first_tag: int = 0):
        if num_pages < 0:
            raise ValueError("num_pages must be >= 0")
        self.num_pages = int(num_pages)
        self.tags = np.full(self.num_pages, first_tag, dtype=np.uint32)
        ids = np.arange(self.num_pages, dtype=np.int32)
        if order == "shuffled":
            rng(seed, 0x9001).shuffle(ids)
        elif order != "sequential":
            raise ValueError("order must be 'shuffled' or 'sequential'")
        self._free = collections.deque(int(i) for i in ids)

    @property
    def free_pages(self) -> int:
        return len(self._free)

    def alloc(self, n: int):
        """Take n pages from the free list; returns (page ids, their new tags)."""
        if n > len(self._free):
            raise PoolExhausted(f"need {n} pages, {len(self._free)} free of {self.num_pages}")
        pages = np.array([self._free.popleft() for _ in range(n)], dtype=np.int32)
        self.tags[pages] += np.uint32(1)
        return pages, self.tags[pages].copy()

    def release(self, pages: Sequence[int]) -> None:
        for p in pages:
            self._free.append(int(p))

    def reallocate(self, page: int) -> None:
        """Page is freed by its owner and immediately handed to another request
        (its generation tag changes)."""
        self.tags[page] += np.uint32(1)


@dataclasses.dataclass
class PagedBatch:
    """Per-request mapping of logical pages onto the shared physical pool."""
    page_size: int
    page_table: np.ndarray      # int32 [B][max_pages]; -1 where unused
    context_lens: np.ndarray    # int32 [B]; tokens attended, including this step's token
    expected_tags: np.ndarray   # uint32 [B][max_pages]; tag recorded at allocation

    @property
    def batch(self) -> int:
        return int(self.page_table.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])


def pages_needed(length: int, page_size: int) -> int:
    return (int(length) + page_size - 1) // page_size


def allocate_batch(pool: PagePool, context_lens: Sequence[int], page_size: int,
                   max_pages: Optional[int] = None) -> PagedBatch:
    """Allocate ceil(L_b / P) pages for every request, in request order."""
    lens = np.asarray(context_lens, dtype=np.int32)
    need = [pages_needed(L, page_size) for L in lens]
    maxp = int(max_pages if max_pages is not None else max(need + [1]))
    B = len(lens)
    table = np.full((B, maxp), -1, dtype=np.int32)
    tags = np.zeros((B, maxp), dtype=np.uint32)
    for b, n in enumerate(need):
        if n > maxp:
            raise ValueError(f"request {b} needs {n} pages > max_pages {maxp}")
        pages, t = pool.alloc(n)
        table[b, :n] = pages
        tags[b, :n] = t
    return PagedBatch(page_size, table, lens, tags)


def make_stale(pool: PagePool, batch: PagedBatch, b: int, i: int) -> None:
    """Logical page i of request b is reallocated to another owner behind the
    request's back: the physical page's tag moves on, the request keeps the
    tag it recorded."""
    pool.reallocate(int(batch.page_table[b, i]))


# ----------------------------------------------------------------------------
# named workloads
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    page_size: int
    min_len: int
    max_len: int                  # lengths uniform in [min_len, max_len]
    pool_factor: float = 1.0      # pool pages = factor * pages required (ignored if pool_pages)
    pool_pages: Optional[int] = None
    outlier_frac: float = 0.0
    outlier_mult: float = 20.0
    num_splits: int = 0           # 0 = library's choice
    stale_requests: int = 0
    # peaked-softmax and dynamic-range recipes (device inputs only):
    q_mult: float = 1.0           # q ~ N(0, 1) * q_mult before bf16 rounding
    k_log2: int = 0               # K data times 2^k_log2 (exact on bf16 values)
    v_log2: int = 0               # V data times 2^v_log2
    v_bias: float = 0.0           # added to the even head dims of V before rounding
    needle_gap: float = 0.0       # > 0: needle tokens (below) score this many nats
                                  # above a near-flat background

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads


def kv_page_bytes(kv_heads: int, page_size: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes one physical page occupies in the K and V pools together."""
    return 2 * kv_heads * page_size * head_dim * elem_bytes


def pages_in_budget(budget_bytes: int, kv_heads: int, page_size: int, head_dim: int,
                    elem_bytes: int) -> int:
    return budget_bytes // kv_page_bytes(kv_heads, page_size, head_dim, elem_bytes)


# the memory budget of the concurrency sweep: exactly 32 bf16 requests of 16k tokens
SWEEP_BUDGET_BYTES = 32 * 256 * kv_page_bytes(8, 64, 128, 2)  # 2 GiB

WORKLOADS = {
    # one request, 4 query heads on 4 KV heads, head_dim 64, 256 tokens in 16-token pages
    "tiny_mha_d64_256": Workload("tiny_mha_d64_256", 1, 4, 4, 64, 16, 256, 256, pool_pages=32),
    # 8 requests, GQA 32/8, head_dim 128, 4096 tokens, 16-token pages, 1% outliers x20
    "gqa4_4k_outliers": Workload("gqa4_4k_outliers", 8, 32, 8, 128, 16, 4096, 4096,
                                 pool_factor=1.25, outlier_frac=0.01, outlier_mult=20.0),
    # 32 requests, GQA 64/8, lengths uniform in [1024, 32768], 64-token pages, fragmented pool
    "gqa8_ragged_32k": Workload("gqa8_ragged_32k", 32, 64, 8, 128, 64, 1024, 32768,
                                pool_factor=1.25),
    # concurrency sweep point: B requests of 16384 tokens, GQA 64/8, 64-token pages
    "gqa8_16k_b64": Workload("gqa8_16k_b64", 64, 64, 8, 128, 64, 16384, 16384,
                             pool_pages=pages_in_budget(SWEEP_BUDGET_BYTES, 8, 64, 128, 1)),
    # 4 requests of 262144 tokens, GQA 64/8, 64 splits, one request with a stale tag
    "gqa8_256k_b4": Workload("gqa8_256k_b4", 4, 64, 8, 128, 64, 262144, 262144,
                             pool_pages=16384, num_splits=64, stale_requests=1),
}


def sweep_workload(batch: int, kv_dtype_bytes: int) -> Workload:
    """Concurrency-sweep point: B x 16384 tokens in the 2 GiB budget (holds
    64 e4m3 requests or 32 bf16 requests)."""
    return Workload(f"gqa8_16k_b{batch}", batch, 64, 8, 128, 64, 16384, 16384,
                    pool_pages=pages_in_budget(SWEEP_BUDGET_BYTES, 8, 64, 128, kv_dtype_bytes))


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields changed (used for small test sizes)."""
    return dataclasses.replace(w, **changes)


@dataclasses.dataclass
class DecodeInputs:
    """Everything one decode step needs, on the host."""
    workload: Workload
    seed: int
    q: np.ndarray                 # uint16 bf16 [B][Hq][D]
    k_tokens: List[np.ndarray]    # per request uint16 bf16 [L_b][Hkv][D]; last row is this step's token
    v_tokens: List[np.ndarray]
    k_scale: np.ndarray           # float32 [Hkv]
    v_scale: np.ndarray
    pool: PagePool
    batch: PagedBatch
    stale: List[int]              # requests given a stale tag

    @property
    def num_pages(self) -> int:
        return self.pool.num_pages

    def k_new(self) -> np.ndarray:
        return np.stack([k[-1] for k in self.k_tokens])

    def v_new(self) -> np.ndarray:
        return np.stack([v[-1] for v in self.v_tokens])

    def history(self, b: int):
        """(k, v) of the tokens before this step's token for request b."""
        return self.k_tokens[b][:-1], self.v_tokens[b][:-1]


def stale_requests(w: Workload, seed: int, batch: int) -> List[int]:
    """The requests of a batch that get a stale tag (sorted)."""
    if not w.stale_requests:
        return []
    pick = rng(seed, 5).choice(batch, size=min(w.stale_requests, batch), replace=False)
    return sorted(int(x) for x in pick)


def context_lengths(w: Workload, seed: int) -> np.ndarray:
    if w.min_len == w.max_len:
        return np.full(w.batch, w.max_len, dtype=np.int32)
    return rng(seed, 3).integers(w.min_len, w.max_len + 1, size=w.batch).astype(np.int32)


def make_decode_inputs(w: Workload, seed: int, lengths: Optional[Sequence[int]] = None,
                       pool_order: str = "shuffled") -> DecodeInputs:
    """Draw a full decode step for workload w (host arrays; seeded)."""
    lens = np.asarray(lengths if lengths is not None else context_lengths(w, seed), dtype=np.int32)
    B, Hq, Hkv, D, P = len(lens), w.q_heads, w.kv_heads, w.head_dim, w.page_size
    need = sum(pages_needed(L, P) for L in lens)
    # a fixed budget (pool_pages) is never enlarged: requests that do not fit
    # raise PoolExhausted, the capacity ceiling of that budget
    num_pages = w.pool_pages if w.pool_pages is not None else max(need, int(math.ceil(need * w.pool_factor)))
    pool = PagePool(num_pages, seed=seed, order=pool_order)
    batch = allocate_batch(pool, lens, P)
    q, _ = normal_bf16(rng(seed, 2), (B, Hq, D))
    ks, vs = [], []
    k_amax = np.zeros(Hkv, np.float32)
    v_amax = np.zeros(Hkv, np.float32)
    for b in range(B):
        g = rng(seed, 1, b)
        k = np.empty((int(lens[b]), Hkv, D), np.uint16)
        v = np.empty((int(lens[b]), Hkv, D), np.uint16)
        for h in range(Hkv):
            k[:, h, :], ka = normal_bf16(g, (int(lens[b]), D), w.outlier_frac, w.outlier_mult)
            v[:, h, :], va = normal_bf16(g, (int(lens[b]), D), w.outlier_frac, w.outlier_mult)
            k_amax[h] = max(k_amax[h], ka)
            v_amax[h] = max(v_amax[h], va)
        ks.append(k)
        vs.append(v)
    stale = stale_requests(w, seed, B)
    for b in stale:
        i = int(rng(seed, 6, b).integers(0, pages_needed(lens[b], P)))
        make_stale(pool, batch, b, i)
    return DecodeInputs(w, seed, q, ks, vs, fp8_scale_from_amax(k_amax),
                        fp8_scale_from_amax(v_amax), pool, batch, stale)


# ----------------------------------------------------------------------------
# the same recipe drawn on the GPU (for full-size workloads)
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class DeviceDecodeInputs:
    """A decode step drawn with torch's generator on the GPU.  Token data is
    [B][Tmax][Hkv][D] bf16 (row L_b - 1 is this step's token; rows past L_b
    are zero); scales are fp32 [Hkv] on the device and on the host."""
    workload: Workload
    seed: int
    q: "object"            # torch bf16 [B][Hq][D]
    k_tokens: "object"     # torch bf16 [B][Tmax][Hkv][D]
    v_tokens: "object"
    k_scale: np.ndarray
    v_scale: np.ndarray
    pool: PagePool
    batch: PagedBatch
    stale: List[int]

    @property
    def num_pages(self) -> int:
        return self.pool.num_pages


def _torch_gen(device, seed: int, *stream: int):
    import torch
    ss = np.random.SeedSequence([int(seed), *map(int, stream)])
    g = torch.Generator(device=device)
    g.manual_seed(int(ss.generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF))
    return g


def _device_normal_bf16(g, shape, device, outlier_frac, outlier_mult):
    """N(0,1) -> bf16 (nearest even), outliers after the bulk amax; returns
    (bf16 tensor, per-head bulk amax over all but the head axis (axis -2))."""
    import torch
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    bulk = x.to(torch.bfloat16)
    amax = bulk.abs().float().amax(dim=tuple(i for i in range(len(shape)) if i != len(shape) - 2))
    if outlier_frac > 0.0:
        mask = torch.rand(shape, generator=g, device=device, dtype=torch.float32) < outlier_frac
        bulk = torch.where(mask, x * outlier_mult, x).to(torch.bfloat16)
    return bulk, amax


NEEDLE_EVERY, NEEDLE_SPAN = 32, 256   # needle tokens: every 32nd token of the first 256


def _needle_shape(w: Workload, q, k, v, L: int):
    """The needle recipe for one request (in place, fp32 [L][Hkv][D] K/V and
    fp32 [Hq][D] q): the query heads of a KV head share one query vector;
    background keys are small (N(0, 2^-12)), so their scores are nearly
    equal; tokens 0, 32, .., 224 are needles whose key is the group's query
    direction scaled so that its score is needle_gap nats above the
    background's, with V near zero (N(0, 2^-12)).  Every wave tile of the
    first 256 tokens then holds a needle, and each later token weighs about
    exp(-needle_gap) of a needle."""
    import torch
    G, D = w.group, w.head_dim
    qg = q.view(w.kv_heads, G, D)[:, :1, :].expand(-1, G, -1).clone()
    q.copy_(qg.reshape(w.q_heads, D))
    k.mul_(2.0 ** -6)
    sm = 1.0 / math.sqrt(D)
    qv = q.view(w.kv_heads, G, D)[:, 0, :]                        # [Hkv][D]
    needle_k = qv * (w.needle_gap / sm) / (qv * qv).sum(-1, keepdim=True)
    idx = torch.arange(0, min(L, NEEDLE_SPAN), NEEDLE_EVERY, device=k.device)
    k[idx] = needle_k.to(k.dtype)
    v[idx] = v[idx] * 2.0 ** -6


def _device_kv(w: Workload, g, L: int, device, q=None):
    """One request's K and V ([L][Hkv][D] bf16) by the workload's recipe, and
    the per-head amax of the data the scales come from (the bulk before
    outliers)."""
    import torch
    shaped = w.v_bias != 0.0 or w.needle_gap > 0.0 or w.k_log2 != 0 or w.v_log2 != 0
    kb, ka = _device_normal_bf16(g, (L, w.kv_heads, w.head_dim), device, w.outlier_frac, w.outlier_mult)
    vb, va = _device_normal_bf16(g, (L, w.kv_heads, w.head_dim), device, w.outlier_frac, w.outlier_mult)
    if not shaped:
        return kb, ka, vb, va
    if w.outlier_frac > 0.0:
        raise ValueError("outliers and the peaked recipes are not combined")
    k, v = kb.float(), vb.float()
    if w.v_bias != 0.0:
        v[..., 0::2] += w.v_bias
    if w.needle_gap > 0.0:
        _needle_shape(w, q, k, v, L)
    kb = (k.to(torch.bfloat16) * 2.0 ** w.k_log2)   # power-of-two scaling: exact
    vb = (v.to(torch.bfloat16) * 2.0 ** w.v_log2)
    ka = kb.abs().float().amax(dim=(0, 2))
    va = vb.abs().float().amax(dim=(0, 2))
    return kb, ka, vb, va


def make_device_decode_inputs(w: Workload, seed: int, device="cuda",
                              lengths: Optional[Sequence[int]] = None,
                              pool_order: str = "shuffled") -> DeviceDecodeInputs:
    """Draw a decode step for workload w directly on the GPU (seeded per request)."""
    import torch
    lens = np.asarray(lengths if lengths is not None else context_lengths(w, seed), dtype=np.int32)
    B, Hq, Hkv, D, P = len(lens), w.q_heads, w.kv_heads, w.head_dim, w.page_size
    need = sum(pages_needed(L, P) for L in lens)
    # a fixed budget (pool_pages) is never enlarged: requests that do not fit
    # raise PoolExhausted, the capacity ceiling of that budget
    num_pages = w.pool_pages if w.pool_pages is not None else max(need, int(math.ceil(need * w.pool_factor)))
    pool = PagePool(num_pages, seed=seed, order=pool_order)
    batch = allocate_batch(pool, lens, P)
    T = int(lens.max()) if B else 1
    qg = _torch_gen(device, seed, 2)
    if w.q_mult == 1.0 and w.needle_gap == 0.0:
        q, _ = _device_normal_bf16(qg, (B, Hq, D), device, 0.0, 1.0)
        qf = None
    else:
        qf = torch.randn((B, Hq, D), generator=qg, device=device, dtype=torch.float32) * w.q_mult
    k = torch.zeros((B, T, Hkv, D), dtype=torch.bfloat16, device=device)
    v = torch.zeros_like(k)
    k_amax = torch.zeros(Hkv, dtype=torch.float32, device=device)
    v_amax = torch.zeros_like(k_amax)
    for b in range(B):
        L = int(lens[b])
        g = _torch_gen(device, seed, 1, b)
        kb, ka, vb, va = _device_kv(w, g, L, device, None if qf is None else qf[b])
        k[b, :L] = kb
        v[b, :L] = vb
        k_amax = torch.maximum(k_amax, ka)
        v_amax = torch.maximum(v_amax, va)
    if qf is not None:
        q = qf.to(torch.bfloat16)
    stale = stale_requests(w, seed, B)
    for b in stale:
        i = int(rng(seed, 6, b).integers(0, pages_needed(lens[b], P)))
        make_stale(pool, batch, b, i)
    return DeviceDecodeInputs(w, seed, q, k, v, fp8_scale_from_amax(k_amax.cpu().numpy()),
                              fp8_scale_from_amax(v_amax.cpu().numpy()), pool, batch, stale)
