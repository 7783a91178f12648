"""Device-side set-up around the library: upload a batch, build a cache.

Used by the tests and the bench.  The cache is built with the library's own
kv_quant_fill (the prefill-to-decode hand-off) for every token but this
step's, which kv_quant_append writes as part of the decode step.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import inputs as I
from . import ops

FP8_NAN_CODE = 0x7F
BF16_NAN_BITS = 0x7FC0


@dataclasses.dataclass
class DeviceStep:
    """Device tensors of one decode step."""
    cache: ops.PagedKVCache
    batch: ops.DecodeBatch           # req_status unset (no-op tracker)
    page_tags: torch.Tensor          # int32 view of the uint32 tags [num_pages]
    expected_tags: torch.Tensor      # int32 view [B][max_pages]
    q: torch.Tensor                  # bf16 [B][Hq][D]
    k_new: torch.Tensor              # bf16 [B][Hkv][D]
    v_new: torch.Tensor


def upload_batch(batch: I.PagedBatch, pool: I.PagePool, device):
    pt = torch.from_numpy(np.ascontiguousarray(batch.page_table)).to(device)
    lens = torch.from_numpy(np.ascontiguousarray(batch.context_lens)).to(device)
    tags = torch.from_numpy(np.ascontiguousarray(pool.tags).view(np.int32)).to(device)
    exp = torch.from_numpy(np.ascontiguousarray(batch.expected_tags).view(np.int32)).to(device)
    return ops.DecodeBatch(pt, lens), tags, exp


def poison_(cache: ops.PagedKVCache) -> None:
    """Fill the whole pool with NaN codes, as stale memory of other owners."""
    if cache.kv_dtype == ops.KV_FP8_E4M3:
        cache.k_pool.fill_(FP8_NAN_CODE)
        cache.v_pool.fill_(FP8_NAN_CODE)
    else:
        cache.k_pool.view(torch.int16).fill_(BF16_NAN_BITS)
        cache.v_pool.view(torch.int16).fill_(BF16_NAN_BITS)


def new_cache(w: I.Workload, num_pages: int, kv_dtype: int, device, k_scale=None, v_scale=None,
              poison: bool = True) -> ops.PagedKVCache:
    ks = vs = None
    if kv_dtype == ops.KV_FP8_E4M3:
        ks = torch.from_numpy(np.asarray(k_scale, np.float32)).to(device)
        vs = torch.from_numpy(np.asarray(v_scale, np.float32)).to(device)
    cache = ops.PagedKVCache.allocate(num_pages, w.kv_heads, w.page_size, w.head_dim, kv_dtype,
                                      device, ks, vs)
    if poison:
        poison_(cache)
    return cache


def fill_history(cache: ops.PagedKVCache, batch: ops.DecodeBatch, k_tokens: torch.Tensor,
                 v_tokens: torch.Tensor, context_lens: np.ndarray, chunk: int = 8) -> None:
    """kv_quant_fill of tokens [0, L_b - 1) of every request, a few requests
    per call ([B][T][Hkv][D] sources)."""
    B = batch.batch
    dev = cache.device
    for b0 in range(0, B, chunk):
        b1 = min(B, b0 + chunk)
        sub = ops.DecodeBatch(batch.page_table[b0:b1].contiguous(),
                              batch.context_lens[b0:b1].contiguous())
        counts = np.maximum(np.asarray(context_lens[b0:b1], np.int32) - 1, 0)
        T = max(1, int(counts.max()))
        start = torch.zeros(b1 - b0, dtype=torch.int32, device=dev)
        count = torch.from_numpy(counts).to(dev)
        ops.kv_quant_fill(cache, sub, start, count, k_tokens[b0:b1, :T].contiguous(),
                          v_tokens[b0:b1, :T].contiguous())


def host_tokens_to_device(inp: I.DecodeInputs, device):
    """Pad the host per-request token arrays into [B][Tmax][Hkv][D] bf16."""
    w = inp.workload
    B = inp.batch.batch
    T = max(int(k.shape[0]) for k in inp.k_tokens)
    k = np.zeros((B, T, w.kv_heads, w.head_dim), np.uint16)
    v = np.zeros_like(k)
    for b in range(B):
        n = inp.k_tokens[b].shape[0]
        k[b, :n] = inp.k_tokens[b]
        v[b, :n] = inp.v_tokens[b]
    to = lambda a: torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return to(k), to(v)


def bf16_tensor(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).to(device).view(torch.bfloat16)


def build_step(inp, kv_dtype: int, device, poison: bool = True) -> DeviceStep:
    """Device cache holding every token but this step's, plus the step's inputs.
    inp is a host DecodeInputs or a DeviceDecodeInputs."""
    w = inp.workload
    cache = new_cache(w, inp.num_pages, kv_dtype, device, inp.k_scale, inp.v_scale, poison)
    batch, tags, exp = upload_batch(inp.batch, inp.pool, device)
    if isinstance(inp, I.DecodeInputs):
        k, v = host_tokens_to_device(inp, device)
        q = bf16_tensor(inp.q, device)
    else:
        k, v, q = inp.k_tokens, inp.v_tokens, inp.q
    fill_history(cache, batch, k, v, inp.batch.context_lens)
    lens = torch.from_numpy(np.asarray(inp.batch.context_lens, np.int64) - 1).to(device)
    idx = lens.clamp(min=0).view(-1, 1, 1, 1).expand(-1, 1, w.kv_heads, w.head_dim)
    k_new = torch.gather(k, 1, idx).squeeze(1).contiguous()
    v_new = torch.gather(v, 1, idx).squeeze(1).contiguous()
    return DeviceStep(cache, batch, tags, exp, q, k_new, v_new)


def decode_step(step: DeviceStep, sm_scale: float, num_splits: int = 0, check: bool = True,
                workspace: Optional[torch.Tensor] = None, out=None, lse=None,
                fused: bool = False, append_in_attention: bool = False):
    """One decode step of the path: tag check (unless check=False: no-op
    tracker), append, attention (with its split-K combine).  fused: the check
    runs inside the append launch (kv_quant_append_checked).
    append_in_attention: the append runs inside the attention launch."""
    status = None
    if append_in_attention:
        if check:
            status = ops.page_tag_check(step.batch, step.cache.page_size, step.page_tags,
                                        step.expected_tags)
        b = step.batch.with_status(status)
        o, l = ops.paged_decode_attn(step.cache, b, step.q, sm_scale, num_splits, workspace, out, lse,
                                     k_new=step.k_new, v_new=step.v_new)
        return o, l, status
    if fused:
        status = ops.kv_quant_append_checked(step.cache, step.batch, step.page_tags,
                                             step.expected_tags, step.k_new, step.v_new)
        b = step.batch.with_status(status)
    else:
        if check:
            status = ops.page_tag_check(step.batch, step.cache.page_size, step.page_tags,
                                        step.expected_tags)
        b = step.batch.with_status(status)
        ops.kv_quant_append(step.cache, b, step.k_new, step.v_new)
    o, l = ops.paged_decode_attn(step.cache, b, step.q, sm_scale, num_splits, workspace, out, lse)
    return o, l, status
