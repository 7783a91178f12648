// api.hip -- the C ABI declared in include/pafp8.h.
//
// Validation happens here, on the host, before anything is launched; a
// rejected call returns a status and a message (pafp8_last_error) and touches
// no device state.  Validation makes no HIP call, so it can be exercised on a
// machine without a GPU.
#include "pafp8.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "pafp8_internal.hpp"

namespace {

thread_local char g_err[512];

pafp8_status fail(pafp8_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

pafp8_status ok()
{
    g_err[0] = '\0';
    return PAFP8_OK;
}

pafp8_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess)
        return ok();
    return fail(PAFP8_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int log2_exact(int v)
{
    for (int k = 0; k < 31; ++k)
        if (v == (1 << k))
            return k;
    return -1;
}

// largest W of a balanced launch (num_splits = -W)
constexpr int32_t kMaxBalancedGroups = 65536;

size_t align16_up(size_t n) { return (n + 15) & ~size_t{15}; }

bool page_size_ok(int P) { return P == 16 || P == 32 || P == 64 || P == 128 || P == 256; }

pafp8_status check_batch(const pafp8_batch *b, bool need_lens)
{
    if (b == nullptr)
        return fail(PAFP8_EINVAL, "batch descriptor is NULL");
    if (b->batch < 0)
        return fail(PAFP8_EINVAL, "batch = %d < 0", b->batch);
    if (b->max_pages_per_req < 1)
        return fail(PAFP8_EINVAL, "max_pages_per_req = %d < 1", b->max_pages_per_req);
    if (b->batch > 0 && b->page_table == nullptr)
        return fail(PAFP8_EINVAL, "page_table is NULL");
    if (need_lens && b->batch > 0 && b->context_lens == nullptr)
        return fail(PAFP8_EINVAL, "context_lens is NULL");
    return PAFP8_OK;
}

pafp8_status check_cache(const pafp8_cache *c, int want_dtype)
{
    if (c == nullptr)
        return fail(PAFP8_EINVAL, "cache descriptor is NULL");
    if (c->kv_dtype != PAFP8_KV_FP8_E4M3 && c->kv_dtype != PAFP8_KV_BF16)
        return fail(PAFP8_EINVAL, "kv_dtype = %d is not a known pool type", c->kv_dtype);
    if (want_dtype >= 0 && c->kv_dtype != want_dtype)
        return fail(PAFP8_EINVAL, "pool type %s does not match this entry point (%s)",
                    c->kv_dtype == PAFP8_KV_BF16 ? "bf16" : "e4m3",
                    want_dtype == PAFP8_KV_BF16 ? "bf16" : "e4m3");
    if (c->num_pages < 1)
        return fail(PAFP8_EINVAL, "num_pages = %d < 1", c->num_pages);
    if (!page_size_ok(c->page_size))
        return fail(PAFP8_EUNSUPPORTED, "page_size = %d (supported: 16, 32, 64, 128, 256)",
                    c->page_size);
    if (c->num_kv_heads < 1)
        return fail(PAFP8_EINVAL, "num_kv_heads = %d < 1", c->num_kv_heads);
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(PAFP8_EUNSUPPORTED, "head_dim = %d (supported: 64, 128)", c->head_dim);
    if (c->k_pool == nullptr || c->v_pool == nullptr)
        return fail(PAFP8_EINVAL, "k_pool or v_pool is NULL");
    if (!aligned16(c->k_pool) || !aligned16(c->v_pool))
        return fail(PAFP8_EINVAL, "k_pool and v_pool must be 16-byte aligned");
    if (c->kv_dtype == PAFP8_KV_FP8_E4M3 && (c->k_scale == nullptr || c->v_scale == nullptr))
        return fail(PAFP8_EINVAL, "e4m3 pools need k_scale and v_scale");
    const int64_t elems = static_cast<int64_t>(c->num_pages) * c->num_kv_heads * c->page_size *
                          c->head_dim;
    if (elems / c->num_pages / c->num_kv_heads != static_cast<int64_t>(c->page_size) * c->head_dim)
        return fail(PAFP8_EINVAL, "pool geometry overflows");
    return PAFP8_OK;
}

pafp8_status check_attn(const pafp8_cache *cache, const pafp8_batch *batch, const uint16_t *q,
                        int32_t Hq, float sm_scale, int32_t S, void *ws, size_t ws_bytes,
                        const float *out, int want_dtype)
{
    pafp8_status st = check_cache(cache, want_dtype);
    if (st != PAFP8_OK)
        return st;
    if ((st = check_batch(batch, true)) != PAFP8_OK)
        return st;
    if (Hq < 1 || Hq % cache->num_kv_heads != 0)
        return fail(PAFP8_EINVAL, "num_q_heads = %d is not a positive multiple of num_kv_heads = %d",
                    Hq, cache->num_kv_heads);
    const int G = Hq / cache->num_kv_heads;
    if (G > 16)
        return fail(PAFP8_EUNSUPPORTED, "query group size %d > 16", G);
    if (!(sm_scale > 0.0f) || sm_scale > 3.0e38f)
        return fail(PAFP8_EINVAL, "sm_scale must be positive and finite");
    if (S < -kMaxBalancedGroups)
        return fail(PAFP8_EINVAL, "num_splits = %d: a balanced launch takes at most %d work-groups per KV head",
                    S, kMaxBalancedGroups);
    if (S < 0 && (static_cast<int64_t>(cache->num_kv_heads) * -S > 0x7FFFFFFF ||
                  static_cast<int64_t>(batch->batch) - S - 1 > 0x7FFFFFFF))
        return fail(PAFP8_EUNSUPPORTED, "a balanced launch of %d work-groups per KV head is too large", -S);
    if (batch->batch > 0 && (q == nullptr || out == nullptr))
        return fail(PAFP8_EINVAL, "q or out is NULL");
    if (batch->batch > 0 && (!aligned16(q) || !aligned16(out)))
        return fail(PAFP8_EINVAL, "q and out must be 16-byte aligned");
    (void)ws;
    (void)ws_bytes;
    return PAFP8_OK;
}

// CU count per device, cached (the only process-wide state besides the
// thread-local error text)
std::mutex g_cu_mu;
std::vector<int> g_cu;

int device_cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 256;
    std::lock_guard<std::mutex> lk(g_cu_mu);
    if (dev >= static_cast<int>(g_cu.size()))
        g_cu.resize(dev + 1, 0);
    if (g_cu[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        g_cu[dev] = n;
    }
    return g_cu[dev];
}

// Scratch of paged_decode_attn_fp8_noalloc: the split-K / balanced partials
// of a call live here instead of in a caller's workspace.  Each GPU the
// library runs on holds its own copy until the process ends.  Host code must
// not pass the array's name to a kernel (on the host it is a stand-in, not a
// device address): the device address comes from hipGetSymbolAddress, once
// per device, and only that address is used.
constexpr size_t kScratchBytes = size_t{16} << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::vector<void *> g_scratch;

// the current device's address of `scratch` (looked up on first use)
pafp8_status scratch_address(void **addr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_status(e, "hipGetDevice");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (dev >= static_cast<int>(g_scratch.size()))
        g_scratch.resize(dev + 1, nullptr);
    if (g_scratch[dev] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (ptr == nullptr)
            return fail(PAFP8_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch[dev] = ptr;
    }
    *addr = g_scratch[dev];
    return PAFP8_OK;
}

pafp8_status attn_impl(const pafp8_cache *cache, const pafp8_batch *batch, const uint16_t *q,
                       int32_t Hq, float sm_scale, int32_t S, void *ws, size_t ws_bytes,
                       float *out, float *lse, hipStream_t stream, int want_dtype,
                       bool append = false, const uint16_t *k_new = nullptr,
                       const uint16_t *v_new = nullptr)
{
    pafp8_status st = check_attn(cache, batch, q, Hq, sm_scale, S, ws, ws_bytes, out, want_dtype);
    if (st != PAFP8_OK)
        return st;
    if (append && batch->batch > 0 && (k_new == nullptr || v_new == nullptr))
        return fail(PAFP8_EINVAL, "k_new or v_new is NULL");
    if (batch->batch == 0)
        return ok();
    if (S == 0)
        S = pafp8_default_num_splits(batch->batch, cache->num_kv_heads, batch->max_pages_per_req,
                                     cache->page_size, 0);
    if (S > batch->max_pages_per_req)
        S = batch->max_pages_per_req;  // more splits than pages would all be empty
    const bool balanced = S < 0;
    const size_t need = pafp8_decode_workspace_bytes(batch->batch, Hq, cache->head_dim, S);
    if (need > 0) {
        if (ws == nullptr || ws_bytes < need)
            return fail(PAFP8_EINVAL, "num_splits = %d needs a workspace of %zu bytes (got %zu)",
                        S, need, ws == nullptr ? size_t{0} : ws_bytes);
        if (!aligned16(ws))
            return fail(PAFP8_EINVAL, "workspace must be 16-byte aligned");
    }
    pafp8::AttnParams p{};
    p.k_pool = static_cast<const uint8_t *>(cache->k_pool);
    p.v_pool = static_cast<const uint8_t *>(cache->v_pool);
    p.k_scale = cache->kv_dtype == PAFP8_KV_FP8_E4M3 ? cache->k_scale : nullptr;
    p.v_scale = cache->kv_dtype == PAFP8_KV_FP8_E4M3 ? cache->v_scale : nullptr;
    p.page_table = batch->page_table;
    p.context_lens = batch->context_lens;
    p.req_status = batch->req_status;
    p.q = q;
    p.k_new = append ? k_new : nullptr;
    p.v_new = append ? v_new : nullptr;
    p.out = out;
    p.lse = lse;
    p.num_pages = cache->num_pages;
    p.log2_page = log2_exact(cache->page_size);
    p.num_kv_heads = cache->num_kv_heads;
    p.batch = batch->batch;
    p.max_pages = batch->max_pages_per_req;
    p.num_q_heads = Hq;
    p.group = Hq / cache->num_kv_heads;
    p.num_splits = balanced ? 1 : S;
    p.pages_per_split = balanced ? batch->max_pages_per_req : (batch->max_pages_per_req + S - 1) / S;
    p.bal_groups = balanced ? -S : 0;
    p.sm_scale = sm_scale;
    // Many uniform splits (at least one per wave slot of the GPU: 64
    // partitions of four 256k-token requests, say) run in wave mode: every
    // wave takes one or two whole splits of one (request, KV head) and
    // writes their partial rows itself, so split boundaries cost no barrier.
    // It needs splits of whole tiles (64 e4m3 or 32 bf16 tokens) and pages of
    // at least a tile; the append taken into the launch keeps the work-group
    // mode.
    p.wave_parts = 0;
    p.part_tiles = 0;
    if (!balanced && S > 1 && !append) {
        const int64_t tile = cache->kv_dtype == PAFP8_KV_BF16 ? 32 : 64;
        const int64_t split_tokens = static_cast<int64_t>(p.pages_per_split) * cache->page_size;
        const int64_t units = static_cast<int64_t>(batch->batch) * cache->num_kv_heads * S;
        const int64_t slots = 4 * static_cast<int64_t>(device_cu_count());  // one work-group per CU
        if (cache->page_size >= tile && split_tokens % tile == 0 && units >= slots) {
            // a wave takes at most two splits: the rows of the first wait in
            // registers until the second is done
            p.wave_parts = units >= 2 * slots ? 2 : 1;
            p.part_tiles = static_cast<int32_t>(split_tokens / tile);
        }
    }
    if (balanced) {
        const size_t R = static_cast<size_t>(batch->batch) + static_cast<size_t>(-S) - 1;  // B + W - 1
        const size_t o_bytes = align16_up(static_cast<size_t>(Hq) * R * cache->head_dim * sizeof(float));
        const size_t l_bytes = align16_up(static_cast<size_t>(Hq) * R * sizeof(float));
        p.part_o = static_cast<float *>(ws);
        p.part_lse = reinterpret_cast<float *>(static_cast<char *>(ws) + o_bytes);
        p.bal_prefix = reinterpret_cast<int64_t *>(static_cast<char *>(ws) + o_bytes + l_bytes);
    } else if (S > 1) {
        p.part_o = static_cast<float *>(ws);
        p.part_lse = p.part_o + static_cast<size_t>(batch->batch) * Hq * S * cache->head_dim;
    }
    hipError_t e = pafp8::launch_decode_attn(cache->kv_dtype == PAFP8_KV_BF16, cache->head_dim, p,
                                             stream);
    if (e != hipSuccess)
        return hip_status(e, "paged_decode_attn launch");
    if (balanced) {
        e = pafp8::launch_bal_combine(p.part_o, p.part_lse, p.bal_prefix, batch->batch, Hq, -S,
                                      cache->head_dim, batch->req_status, batch->context_lens,
                                      batch->max_pages_per_req, p.log2_page, out, lse, stream);
        if (e != hipSuccess)
            return hip_status(e, "balanced combine launch");
    } else if (S > 1) {
        e = pafp8::launch_splitk_combine(p.part_o, p.part_lse, batch->batch, Hq, S,
                                         cache->head_dim, batch->req_status, out, lse, stream);
        if (e != hipSuccess)
            return hip_status(e, "splitk_combine launch");
    }
    return ok();
}

pafp8_status write_impl(const pafp8_cache *cache, const pafp8_batch *batch, bool append,
                        const int32_t *start, const int32_t *count, int32_t T,
                        const uint16_t *k_src, const uint16_t *v_src, hipStream_t stream,
                        const uint32_t *page_tags = nullptr, const uint32_t *expected_tags = nullptr,
                        int32_t *status_out = nullptr, bool checked = false)
{
    pafp8_status st = check_cache(cache, -1);
    if (st != PAFP8_OK)
        return st;
    if ((st = check_batch(batch, append)) != PAFP8_OK)
        return st;
    if (batch->batch == 0)
        return ok();
    if (k_src == nullptr || v_src == nullptr)
        return fail(PAFP8_EINVAL, "source K/V is NULL");
    if (checked && (page_tags == nullptr || expected_tags == nullptr || status_out == nullptr))
        return fail(PAFP8_EINVAL, "page_tags, expected_tags or req_status_out is NULL");
    if (!append) {
        if (start == nullptr || count == nullptr)
            return fail(PAFP8_EINVAL, "token_start or token_count is NULL");
        if (T < 1)
            return fail(PAFP8_EINVAL, "src_tokens = %d < 1", T);
        if (!aligned16(k_src) || !aligned16(v_src))
            return fail(PAFP8_EINVAL, "k_src and v_src must be 16-byte aligned");
        // the fill addresses 16 source rows from one base with 32-bit offsets
        if (static_cast<int64_t>(cache->num_kv_heads) * cache->head_dim > (int64_t{1} << 25))
            return fail(PAFP8_EUNSUPPORTED, "num_kv_heads * head_dim = %lld exceeds 2^25 for kv_quant_fill",
                        static_cast<long long>(cache->num_kv_heads) * cache->head_dim);
    }
    pafp8::WriteParams p{};
    p.k_pool = static_cast<uint8_t *>(cache->k_pool);
    p.v_pool = static_cast<uint8_t *>(cache->v_pool);
    p.k_scale = cache->k_scale;
    p.v_scale = cache->v_scale;
    p.page_table = batch->page_table;
    p.req_status = batch->req_status;
    p.context_lens = append ? batch->context_lens : nullptr;
    p.token_start = start;
    p.token_count = count;
    p.k_src = k_src;
    p.v_src = v_src;
    p.src_tokens = append ? 1 : T;
    p.num_pages = cache->num_pages;
    p.log2_page = log2_exact(cache->page_size);
    p.num_kv_heads = cache->num_kv_heads;
    p.batch = batch->batch;
    p.max_pages = batch->max_pages_per_req;
    if (checked) {
        p.req_status = nullptr;
        p.page_tags = page_tags;
        p.expected_tags = expected_tags;
        p.status_out = status_out;
    }
    return hip_status(pafp8::launch_kv_write(cache->kv_dtype == PAFP8_KV_BF16, cache->head_dim, p,
                                             stream),
                      checked ? "kv_quant_append_checked launch"
                              : append ? "kv_quant_append launch" : "kv_quant_fill launch");
}

}  // namespace

extern "C" {

pafp8_status page_tag_check(const pafp8_batch *batch, int32_t page_size,
                            const uint32_t *page_tags, int32_t num_pages,
                            const uint32_t *expected_tags, int32_t *req_status_out,
                            hipStream_t stream)
{
    pafp8_status st = check_batch(batch, true);
    if (st != PAFP8_OK)
        return st;
    if (!page_size_ok(page_size))
        return fail(PAFP8_EUNSUPPORTED, "page_size = %d (supported: 16, 32, 64, 128, 256)",
                    page_size);
    if (num_pages < 0)
        return fail(PAFP8_EINVAL, "num_pages = %d < 0", num_pages);
    if (batch->batch == 0)
        return ok();
    if (expected_tags == nullptr || req_status_out == nullptr || (num_pages > 0 && page_tags == nullptr))
        return fail(PAFP8_EINVAL, "expected_tags, page_tags or req_status_out is NULL");
    return hip_status(pafp8::launch_tag_check(batch->batch, batch->max_pages_per_req, page_size,
                                              batch->page_table, batch->context_lens,
                                              expected_tags, page_tags, num_pages,
                                              req_status_out, stream),
                      "page_tag_check launch");
}

pafp8_status kv_quant_append(const pafp8_cache *cache, const pafp8_batch *batch,
                             const uint16_t *k_new, const uint16_t *v_new, hipStream_t stream)
{
    return write_impl(cache, batch, true, nullptr, nullptr, 1, k_new, v_new, stream);
}

pafp8_status kv_quant_append_checked(const pafp8_cache *cache, const pafp8_batch *batch,
                                     const uint32_t *page_tags, const uint32_t *expected_tags,
                                     const uint16_t *k_new, const uint16_t *v_new,
                                     int32_t *req_status_out, hipStream_t stream)
{
    return write_impl(cache, batch, true, nullptr, nullptr, 1, k_new, v_new, stream, page_tags,
                      expected_tags, req_status_out, true);
}

pafp8_status page_tag_realloc(int32_t n, const int32_t *page_ids, const int32_t *owner_req,
                              const int32_t *owner_slot, uint32_t *page_tags, int32_t num_pages,
                              int32_t *page_table, uint32_t *expected_tags, int32_t batch,
                              int32_t max_pages_per_req, hipStream_t stream)
{
    if (n < 0 || num_pages < 0 || batch < 0 || max_pages_per_req < 0)
        return fail(PAFP8_EINVAL, "n, num_pages, batch and max_pages_per_req must be >= 0");
    if (n == 0)
        return ok();
    if (page_ids == nullptr || (num_pages > 0 && page_tags == nullptr))
        return fail(PAFP8_EINVAL, "page_ids or page_tags is NULL");
    if ((owner_req == nullptr) != (owner_slot == nullptr))
        return fail(PAFP8_EINVAL, "owner_req and owner_slot must both be given or both be NULL");
    if (owner_req != nullptr && expected_tags == nullptr)
        return fail(PAFP8_EINVAL, "expected_tags is NULL while owners are given");
    return hip_status(pafp8::launch_tag_realloc(n, page_ids, owner_req, owner_slot, page_tags,
                                                num_pages, page_table, expected_tags, batch,
                                                max_pages_per_req, stream),
                      "page_tag_realloc launch");
}

pafp8_status kv_quant_fill(const pafp8_cache *cache, const pafp8_batch *batch,
                           const int32_t *token_start, const int32_t *token_count,
                           int32_t src_tokens, const uint16_t *k_src, const uint16_t *v_src,
                           hipStream_t stream)
{
    return write_impl(cache, batch, false, token_start, token_count, src_tokens, k_src, v_src,
                      stream);
}

size_t pafp8_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                    int32_t num_splits)
{
    if (batch <= 0 || num_q_heads <= 0 || head_dim <= 0 || num_splits == 0 || num_splits == 1 ||
        num_splits < -kMaxBalancedGroups)
        return 0;
    if (num_splits < 0) {
        // partial rows [Hq][B + W - 1][D], their LSEs, then B + 1 int64
        const size_t W = static_cast<size_t>(-num_splits);
        const size_t rows = static_cast<size_t>(num_q_heads) * (static_cast<size_t>(batch) + W - 1);
        return align16_up(rows * static_cast<size_t>(head_dim) * sizeof(float)) +
               align16_up(rows * sizeof(float)) + (static_cast<size_t>(batch) + 1) * sizeof(int64_t);
    }
    const size_t rows = static_cast<size_t>(batch) * num_q_heads * num_splits;
    return rows * static_cast<size_t>(head_dim) * sizeof(float) + rows * sizeof(float);
}

int32_t pafp8_default_balanced_groups(int32_t num_kv_heads, int32_t num_cus)
{
    if (num_kv_heads <= 0)
        return 1;
    if (num_cus <= 0)
        num_cus = device_cu_count();
    // one work-group per CU
    const int64_t W = (static_cast<int64_t>(num_cus) + num_kv_heads - 1) / num_kv_heads;
    return static_cast<int32_t>(W < 1 ? 1 : (W > kMaxBalancedGroups ? kMaxBalancedGroups : W));
}

int32_t pafp8_default_num_splits(int32_t batch, int32_t num_kv_heads, int32_t max_pages_per_req,
                                 int32_t page_size, int32_t num_cus)
{
    if (batch <= 0 || num_kv_heads <= 0 || max_pages_per_req <= 0 || page_size <= 0)
        return 1;
    if (num_cus <= 0)
        num_cus = device_cu_count();
    // about one work-group per CU (measured best from 4 to 64 requests of
    // 16k-256k tokens on MI355X: more, shorter splits add combine traffic and
    // per-split start-up), without splits shorter than 512 tokens, and no
    // split at all below 2048 tokens.  One request on MI355X, e4m3 (bf16):
    // 16k tokens 16.9 us at 16 splits, 16.6 at 32 (21.9, 20.7); 4k tokens 15.6
    // at 4, 13.5 at 8 (19.9, 15.6); 1k tokens 11.9 whole, 13.0 in two halves
    // (the combine launch costs more than the halves save).
    const int64_t units = static_cast<int64_t>(batch) * num_kv_heads;
    int64_t S = (num_cus + units - 1) / units;
    const int64_t tokens = static_cast<int64_t>(max_pages_per_req) * page_size;
    int64_t s_max = tokens >= 2048 ? tokens / 512 : 1;
    if (S > s_max)
        S = s_max;
    if (S > max_pages_per_req)
        S = max_pages_per_req;
    return static_cast<int32_t>(S < 1 ? 1 : S);
}

pafp8_status paged_decode_attn_fp8(const pafp8_cache *cache, const pafp8_batch *batch,
                                   const uint16_t *q, int32_t num_q_heads, float sm_scale,
                                   int32_t num_splits, void *workspace, size_t workspace_bytes,
                                   float *out, float *lse, hipStream_t stream)
{
    return attn_impl(cache, batch, q, num_q_heads, sm_scale, num_splits, workspace,
                     workspace_bytes, out, lse, stream, PAFP8_KV_FP8_E4M3);
}

pafp8_status paged_decode_attn_bf16(const pafp8_cache *cache, const pafp8_batch *batch,
                                    const uint16_t *q, int32_t num_q_heads, float sm_scale,
                                    int32_t num_splits, void *workspace, size_t workspace_bytes,
                                    float *out, float *lse, hipStream_t stream)
{
    return attn_impl(cache, batch, q, num_q_heads, sm_scale, num_splits, workspace,
                     workspace_bytes, out, lse, stream, PAFP8_KV_BF16);
}

size_t pafp8_noalloc_scratch_bytes(void) { return kScratchBytes; }

pafp8_status paged_decode_attn_fp8_noalloc(const pafp8_cache *cache, const pafp8_batch *batch,
                                           const uint16_t *q, int32_t num_q_heads, float sm_scale,
                                           int32_t num_splits, float *out, float *lse,
                                           hipStream_t stream)
{
    pafp8_status st = check_attn(cache, batch, q, num_q_heads, sm_scale, num_splits, nullptr, 0,
                                 out, PAFP8_KV_FP8_E4M3);
    if (st != PAFP8_OK)
        return st;
    if (batch->batch == 0)
        return ok();
    // the split count attn_impl will use, and the partials it needs
    int32_t S = num_splits;
    if (S == 0)
        S = pafp8_default_num_splits(batch->batch, cache->num_kv_heads, batch->max_pages_per_req,
                                     cache->page_size, 0);
    if (S > batch->max_pages_per_req)
        S = batch->max_pages_per_req;
    const size_t need = pafp8_decode_workspace_bytes(batch->batch, num_q_heads, cache->head_dim, S);
    if (need > kScratchBytes)
        return fail(PAFP8_EUNSUPPORTED,
                    "num_splits = %d needs %zu bytes of partials, more than the %zu-byte scratch of "
                    "paged_decode_attn_fp8_noalloc (use paged_decode_attn_fp8 with a workspace)",
                    S, need, kScratchBytes);
    void *ws = nullptr;
    if (need > 0 && (st = scratch_address(&ws)) != PAFP8_OK)
        return st;
    return attn_impl(cache, batch, q, num_q_heads, sm_scale, S, ws, need > 0 ? kScratchBytes : 0,
                     out, lse, stream, PAFP8_KV_FP8_E4M3);
}

pafp8_status paged_decode_attn_fp8_append(const pafp8_cache *cache, const pafp8_batch *batch,
                                          const uint16_t *q, int32_t num_q_heads, float sm_scale,
                                          int32_t num_splits, void *workspace, size_t workspace_bytes,
                                          const uint16_t *k_new, const uint16_t *v_new, float *out,
                                          float *lse, hipStream_t stream)
{
    return attn_impl(cache, batch, q, num_q_heads, sm_scale, num_splits, workspace,
                     workspace_bytes, out, lse, stream, PAFP8_KV_FP8_E4M3, true, k_new, v_new);
}

pafp8_status paged_decode_attn_bf16_append(const pafp8_cache *cache, const pafp8_batch *batch,
                                           const uint16_t *q, int32_t num_q_heads, float sm_scale,
                                           int32_t num_splits, void *workspace, size_t workspace_bytes,
                                           const uint16_t *k_new, const uint16_t *v_new, float *out,
                                           float *lse, hipStream_t stream)
{
    return attn_impl(cache, batch, q, num_q_heads, sm_scale, num_splits, workspace,
                     workspace_bytes, out, lse, stream, PAFP8_KV_BF16, true, k_new, v_new);
}

pafp8_status splitk_combine(const float *part_o, const float *part_lse, int32_t batch,
                            int32_t num_q_heads, int32_t num_splits, int32_t head_dim,
                            const int32_t *req_status, float *out, float *lse,
                            hipStream_t stream)
{
    if (batch < 0 || num_q_heads < 1 || num_splits < 1)
        return fail(PAFP8_EINVAL, "batch, num_q_heads or num_splits out of range");
    if (head_dim < 4 || head_dim > 1024 || head_dim % 4 != 0)
        return fail(PAFP8_EUNSUPPORTED, "head_dim = %d (need a multiple of 4 up to 1024)", head_dim);
    if (batch == 0)
        return ok();
    if (part_o == nullptr || part_lse == nullptr || out == nullptr)
        return fail(PAFP8_EINVAL, "part_o, part_lse or out is NULL");
    if (!aligned16(part_o) || !aligned16(out))
        return fail(PAFP8_EINVAL, "part_o and out must be 16-byte aligned");
    return hip_status(pafp8::launch_splitk_combine(part_o, part_lse, batch, num_q_heads,
                                                   num_splits, head_dim, req_status, out, lse,
                                                   stream),
                      "splitk_combine launch");
}

pafp8_status int4_pack_weights(const uint8_t *w_rowmajor, int32_t N, int32_t K, uint8_t *w_packed,
                               hipStream_t stream)
{
    if (N < 0 || K < 0 || N % 16 != 0 || K % 512 != 0)
        return fail(PAFP8_EUNSUPPORTED, "N = %d, K = %d (need N a multiple of 16, K of 512)", N, K);
    if (N == 0 || K == 0)
        return ok();
    if (w_rowmajor == nullptr || w_packed == nullptr)
        return fail(PAFP8_EINVAL, "w_rowmajor or w_packed is NULL");
    if ((reinterpret_cast<uintptr_t>(w_rowmajor) & 3u) != 0 || !aligned16(w_packed))
        return fail(PAFP8_EINVAL, "w_rowmajor must be 4-byte and w_packed 16-byte aligned");
    return hip_status(pafp8::launch_int4_pack(w_rowmajor, w_packed, N, K, stream),
                      "int4_pack_weights launch");
}

pafp8_status int4_gemv(const uint16_t *x, int32_t M, const uint8_t *w_packed, const uint16_t *scales,
                       int32_t N, int32_t K, float *y, hipStream_t stream)
{
    if (M < 0 || N < 0 || K < 0)
        return fail(PAFP8_EINVAL, "M, N and K must be >= 0");
    if (N % 16 != 0 || K % 512 != 0)
        return fail(PAFP8_EUNSUPPORTED, "N = %d, K = %d (need N a multiple of 16, K of 512)", N, K);
    if (M == 0 || N == 0)
        return ok();
    if (K == 0)
        return fail(PAFP8_EUNSUPPORTED, "K = 0");
    if (x == nullptr || w_packed == nullptr || scales == nullptr || y == nullptr)
        return fail(PAFP8_EINVAL, "x, w_packed, scales or y is NULL");
    if (!aligned16(x) || !aligned16(w_packed))
        return fail(PAFP8_EINVAL, "x and w_packed must be 16-byte aligned");
    // 64 rows of x per launch
    for (int32_t m0 = 0; m0 < M; m0 += 64) {
        const int32_t m = M - m0 < 64 ? M - m0 : 64;
        const hipError_t e = pafp8::launch_int4_gemv(x + static_cast<int64_t>(m0) * K, m, w_packed,
                                                     scales, N, K, y + static_cast<int64_t>(m0) * N,
                                                     device_cu_count(), stream);
        if (e != hipSuccess)
            return hip_status(e, "int4_gemv launch");
    }
    return ok();
}

pafp8_status pafp8_e4m3_encode(const float *x, uint8_t *codes, int64_t n, hipStream_t stream)
{
    if (n < 0)
        return fail(PAFP8_EINVAL, "n = %lld < 0", static_cast<long long>(n));
    if (n == 0)
        return ok();
    if (x == nullptr || codes == nullptr)
        return fail(PAFP8_EINVAL, "x or codes is NULL");
    return hip_status(pafp8::launch_e4m3_encode(x, codes, n, stream), "pafp8_e4m3_encode launch");
}

pafp8_status pafp8_e4m3_decode(const uint8_t *codes, float *out_f32, float *out_via_f16,
                               float *out_via_bf16, int64_t n, hipStream_t stream)
{
    if (n < 0)
        return fail(PAFP8_EINVAL, "n = %lld < 0", static_cast<long long>(n));
    if (n == 0)
        return ok();
    if (codes == nullptr)
        return fail(PAFP8_EINVAL, "codes is NULL");
    return hip_status(pafp8::launch_e4m3_decode(codes, out_f32, out_via_f16, out_via_bf16, n,
                                                stream),
                      "pafp8_e4m3_decode launch");
}

pafp8_status pafp8_stream_read(const void *src, int64_t bytes, int32_t work_groups,
                               uint32_t *sink, int64_t sink_words, hipStream_t stream)
{
    if (bytes < 0 || bytes % pafp8::kStreamReadTile != 0)
        return fail(PAFP8_EINVAL, "bytes = %lld is not a non-negative multiple of %lld",
                    static_cast<long long>(bytes), static_cast<long long>(pafp8::kStreamReadTile));
    if (work_groups < 1)
        return fail(PAFP8_EINVAL, "work_groups = %d < 1", work_groups);
    if (sink_words < static_cast<int64_t>(work_groups) * pafp8::kStreamReadThreads)
        return fail(PAFP8_EINVAL, "sink holds %lld words; work_groups * %d = %lld needed",
                    static_cast<long long>(sink_words), pafp8::kStreamReadThreads,
                    static_cast<long long>(work_groups) * pafp8::kStreamReadThreads);
    if (sink == nullptr || (bytes > 0 && src == nullptr))
        return fail(PAFP8_EINVAL, "src or sink is NULL");
    if (!aligned16(src))
        return fail(PAFP8_EINVAL, "src must be 16-byte aligned");
    return hip_status(pafp8::launch_stream_read(src, bytes, work_groups, sink, stream),
                      "pafp8_stream_read launch");
}

pafp8_status pafp8_stream_read_write(const void *src, int64_t src_bytes, void *dst, int64_t dst_bytes,
                                     int32_t work_groups, hipStream_t stream)
{
    if (src_bytes < 0 || src_bytes % pafp8::kStreamReadTile != 0)
        return fail(PAFP8_EINVAL, "src_bytes = %lld is not a non-negative multiple of %lld",
                    static_cast<long long>(src_bytes), static_cast<long long>(pafp8::kStreamReadTile));
    const int ratio = dst_bytes > 0 && src_bytes % dst_bytes == 0 ? static_cast<int>(src_bytes / dst_bytes) : 0;
    if (src_bytes > 0 && ratio != 1 && ratio != 2 && ratio != 4)
        return fail(PAFP8_EINVAL, "dst_bytes = %lld: src_bytes must be 1, 2 or 4 times it",
                    static_cast<long long>(dst_bytes));
    if (src_bytes == 0 && dst_bytes != 0)
        return fail(PAFP8_EINVAL, "dst_bytes = %lld with src_bytes = 0", static_cast<long long>(dst_bytes));
    if (work_groups < 1)
        return fail(PAFP8_EINVAL, "work_groups = %d < 1", work_groups);
    if (src_bytes == 0)
        return ok();
    if (src == nullptr || dst == nullptr)
        return fail(PAFP8_EINVAL, "src or dst is NULL");
    if (!aligned16(src) || !aligned16(dst))
        return fail(PAFP8_EINVAL, "src and dst must be 16-byte aligned");
    return hip_status(pafp8::launch_stream_read_write(src, src_bytes, dst, ratio, work_groups, stream),
                      "pafp8_stream_read_write launch");
}

const char *pafp8_status_string(pafp8_status status)
{
    switch (status) {
    case PAFP8_OK: return "PAFP8_OK";
    case PAFP8_EINVAL: return "PAFP8_EINVAL";
    case PAFP8_EUNSUPPORTED: return "PAFP8_EUNSUPPORTED";
    case PAFP8_EHIP: return "PAFP8_EHIP";
    default: return "PAFP8_UNKNOWN";
    }
}

const char *pafp8_last_error(void) { return g_err; }

int32_t pafp8_abi_version(size_t *sizeof_cache, size_t *sizeof_batch)
{
    if (sizeof_cache)
        *sizeof_cache = sizeof(pafp8_cache);
    if (sizeof_batch)
        *sizeof_batch = sizeof(pafp8_batch);
    return PAFP8_ABI_VERSION;
}

}  // extern "C"
