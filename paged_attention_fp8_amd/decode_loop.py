"""Multi-step decode with admission over one shared page pool.

Cloudflare, "Smaller, faster, safer: running Kimi and GLM at scale", section
"KV 缓存量化" (KV cache quantization): with the same memory, an e4m3 cache
holds twice the tokens of a bf16 one, so more requests run at once (the post
reports bf16 running out of memory at a concurrency where e4m3 still fits).
Section "共享 KV 缓存保护" (shared KV cache protection): pages are handed from
request to request; each page's tag changes when it is handed on, a request
is checked against the tags it recorded before decode touches the cache, and
a request that fails is terminated.

DecodeLoop runs that cycle on the library's calls only:
  admission   -- the host free list picks pages; page_tag_realloc moves their
                 tags on and writes the request's page-table row and expected
                 tags on the device; kv_quant_fill writes the prompt's K/V
                 (the prefill-to-decode hand-off);
  decode step -- kv_quant_append_checked (tag verdict + append of this step's
                 token) and paged_decode_attn over every slot;
  completion  -- the request's pages go back to the free list;
  termination -- a request whose verdict is not 0 is dropped and its pages
                 are freed.
A request is admitted when pages for its whole length (prompt + decode
tokens) are free, so a running request never waits for a page.  Slots
without a request carry context length 0: the check marks them (bad length)
and the attention call reads nothing for them.

Token data is synthetic (N(0,1) bf16 drawn on the GPU); there are no model
weights.  With record=True the loop keeps a host copy of every K/V token and
query it writes, so tests can rebuild the cache and the attention with the
oracle.
"""
from __future__ import annotations

import collections
import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

from . import ops


@dataclasses.dataclass
class Request:
    rid: int
    prompt_len: int        # tokens handed over from prefill
    decode_len: int        # decode steps to run
    slot: int = -1
    pages: Optional[np.ndarray] = None
    done: int = 0          # decode steps run so far
    admitted_at: int = -1  # loop step of admission
    finished_at: int = -1
    terminated: bool = False

    @property
    def total_len(self) -> int:
        return self.prompt_len + self.decode_len


@dataclasses.dataclass
class StepStats:
    step: int
    active: int            # requests decoded this step
    gpu_ms: float          # append_checked + attention, HIP events
    admitted: int
    finished: int
    terminated: int
    waiting: int


class DecodeLoop:
    def __init__(self, kv_dtype: int, pool_bytes: int, q_heads: int, kv_heads: int, head_dim: int,
                 page_size: int, max_batch: int, max_context: int, device="cuda", seed: int = 0,
                 k_scale=None, v_scale=None, record: bool = False):
        self.kv_dtype = kv_dtype
        self.elem = 1 if kv_dtype == ops.KV_FP8_E4M3 else 2
        self.Hq, self.Hkv, self.D, self.P = q_heads, kv_heads, head_dim, page_size
        self.B = max_batch
        self.maxP = (max_context + page_size - 1) // page_size
        self.num_pages = pool_bytes // (2 * kv_heads * page_size * head_dim * self.elem)
        self.dev = torch.device(device)
        self.gen = torch.Generator(device=self.dev)
        self.gen.manual_seed(seed)
        ks = vs = None
        if kv_dtype == ops.KV_FP8_E4M3:
            # static per-head scales (one fp32 per KV head, K and V apart)
            ks = torch.as_tensor(np.asarray(k_scale, np.float32), device=self.dev)
            vs = torch.as_tensor(np.asarray(v_scale, np.float32), device=self.dev)
        self.cache = ops.PagedKVCache.allocate(self.num_pages, kv_heads, page_size, head_dim,
                                               kv_dtype, self.dev, ks, vs)
        order = np.random.default_rng(seed).permutation(self.num_pages)
        self.free = collections.deque(int(p) for p in order)
        self.page_tags = torch.zeros(self.num_pages, dtype=torch.int32, device=self.dev)
        self.page_table = torch.full((self.B, self.maxP), -1, dtype=torch.int32, device=self.dev)
        self.expected = torch.zeros((self.B, self.maxP), dtype=torch.int32, device=self.dev)
        self.lens = torch.zeros(self.B, dtype=torch.int32, device=self.dev)
        self.status = torch.zeros(self.B, dtype=torch.int32, device=self.dev)
        self.slots: List[Optional[Request]] = [None] * self.B
        self.queue: collections.deque = collections.deque()
        self.finished: List[Request] = []
        self.sm = 1.0 / math.sqrt(head_dim)
        self.splits = ops.default_num_splits(self.B, kv_heads, self.maxP, page_size)
        nws = ops.workspace_bytes(self.B, q_heads, head_dim, self.splits)
        self.ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=self.dev)
        self.out = torch.empty((self.B, q_heads, head_dim), dtype=torch.float32, device=self.dev)
        self.lse = torch.empty((self.B, q_heads), dtype=torch.float32, device=self.dev)
        self.step_no = 0
        self.max_active = 0
        self.record = record
        self.history: Dict[int, Dict[str, list]] = {}
        self.last_q: Optional[torch.Tensor] = None

    # -- request lifecycle ---------------------------------------------------------
    def submit(self, req: Request) -> None:
        if req.total_len > self.maxP * self.P:
            raise ValueError(f"request {req.rid} needs {req.total_len} tokens > {self.maxP * self.P}")
        self.queue.append(req)

    def pages_for(self, req: Request) -> int:
        return (req.total_len + self.P - 1) // self.P

    def _bf16(self, *shape) -> torch.Tensor:
        return torch.randn(*shape, generator=self.gen, device=self.dev, dtype=torch.float32).to(torch.bfloat16)

    def _admit(self) -> int:
        n = 0
        while self.queue:
            req = self.queue[0]
            need = self.pages_for(req)
            slot = next((i for i, r in enumerate(self.slots) if r is None), None)
            if slot is None or need > len(self.free):
                break                  # first come, first served: the head waits
            self.queue.popleft()
            pages = np.array([self.free.popleft() for _ in range(need)], np.int32)
            req.slot, req.pages, req.admitted_at = slot, pages, self.step_no
            self.page_table[slot].fill_(-1)
            ids = torch.from_numpy(pages).to(self.dev)
            owner = torch.full((need,), slot, dtype=torch.int32, device=self.dev)
            idx = torch.arange(need, dtype=torch.int32, device=self.dev)
            ops.page_tag_realloc(ids, self.page_tags, owner, idx, self.page_table, self.expected)
            k = self._bf16(1, req.prompt_len, self.Hkv, self.D)
            v = self._bf16(1, req.prompt_len, self.Hkv, self.D)
            row = ops.DecodeBatch(self.page_table[slot:slot + 1], self.lens[slot:slot + 1])
            zero = torch.zeros(1, dtype=torch.int32, device=self.dev)
            count = torch.full((1,), req.prompt_len, dtype=torch.int32, device=self.dev)
            ops.kv_quant_fill(self.cache, row, zero, count, k, v)
            self.lens[slot] = req.prompt_len
            self.slots[slot] = req
            if self.record:
                self.history[req.rid] = {"k": [k[0].cpu()], "v": [v[0].cpu()]}
            n += 1
        return n

    def _release(self, req: Request, step: int, terminated: bool) -> None:
        self.free.extend(int(p) for p in req.pages)
        self.slots[req.slot] = None
        self.lens[req.slot] = 0
        req.finished_at, req.terminated = step, terminated
        self.finished.append(req)

    def reallocate_behind(self, req: Request, i: int) -> int:
        """Fault injection: page i of a running request is handed to nobody in
        particular while the request still uses it (its tag moves on)."""
        page = int(req.pages[i])
        ids = torch.tensor([page], dtype=torch.int32, device=self.dev)
        ops.page_tag_realloc(ids, self.page_tags)
        return page

    # -- one decode step -------------------------------------------------------------
    def step(self) -> StepStats:
        admitted = self._admit()
        active = [r for r in self.slots if r is not None]
        self.max_active = max(self.max_active, len(active))
        mask = torch.zeros(self.B, dtype=torch.int32)
        for r in active:
            mask[r.slot] = 1
        self.lens += mask.to(self.dev)          # this step's token joins the context
        q = self._bf16(self.B, self.Hq, self.D)
        k_new = self._bf16(self.B, self.Hkv, self.D)
        v_new = self._bf16(self.B, self.Hkv, self.D)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        batch = ops.DecodeBatch(self.page_table, self.lens)
        a.record()
        st = ops.kv_quant_append_checked(self.cache, batch, self.page_tags, self.expected, k_new,
                                         v_new, out=self.status)
        ops.paged_decode_attn(self.cache, batch.with_status(st), q, self.sm, self.splits, self.ws,
                              self.out, self.lse)
        b.record()
        status = st.cpu().numpy()               # synchronises the step
        if self.record:
            for r in active:
                h = self.history[r.rid]
                h["k"].append(k_new[r.slot:r.slot + 1].cpu())
                h["v"].append(v_new[r.slot:r.slot + 1].cpu())
            self.last_q = q.cpu()
        finished = terminated = 0
        for r in active:
            if status[r.slot] != 0:            # the check failed: terminate the request
                self._release(r, self.step_no, True)
                terminated += 1
                continue
            r.done += 1
            if r.done == r.decode_len:
                self._release(r, self.step_no, False)
                finished += 1
        stats = StepStats(self.step_no, len(active), a.elapsed_time(b), admitted, finished,
                          terminated, len(self.queue))
        self.step_no += 1
        return stats

    def tokens_of(self, rid: int):
        """Recorded K/V of a request, bf16 bits [L][Hkv][D] (record=True)."""
        h = self.history[rid]
        k = torch.cat(h["k"]).view(torch.int16).numpy().view(np.uint16)
        v = torch.cat(h["v"]).view(torch.int16).numpy().view(np.uint16)
        return k, v
