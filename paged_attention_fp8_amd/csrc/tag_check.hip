// tag_check.hip -- the batched page-tag integrity check.
//
// Cloudflare, "Smaller, faster, safer: running Kimi and GLM at scale",
// section "共享 KV 缓存保护" (shared KV cache protection): each physical page
// carries a tag that changes when the page is reallocated; the server keeps,
// per request, the pages and tags it expects, and verifies them before decode
// reads the cache; a mismatch terminates that request.  The post runs the
// verification as its own batched pass rather than inside the attention
// kernel (fusing it would race between GPU thread groups); tag_check_kernel
// is that pass: one work-group per request, stream-ordered before append and
// attention, which read its per-request verdict.  (The append kernel can
// also compute the verdict itself: each of its work-groups derives the same
// value from read-only inputs, so nothing races.)
//
// tag_realloc_kernel is the device side of giving a page to a new owner: the
// page's tag moves on, so a request still holding the page with its old tag
// fails the next check.
#include "pafp8_internal.hpp"
#include "tag_verify.hpp"

namespace pafp8 {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void tag_check_kernel(
    int max_pages, int page_size, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ context_lens, const uint32_t *__restrict__ expected_tags,
    const uint32_t *__restrict__ page_tags, int num_pages, int32_t *__restrict__ status)
{
    const int b = blockIdx.x;
    const int flags = request_flags<kThreads>(b, max_pages, page_size, page_table, context_lens,
                                              expected_tags, page_tags, num_pages);
    if (threadIdx.x == 0)
        status[b] = flags;
}

// Device-side reallocation: entry k gives page page_ids[k] a new tag and, if
// its owner lies in the table, records the page and the new tag there.
__global__ __launch_bounds__(kThreads) void tag_realloc_kernel(
    int n, const int32_t *__restrict__ page_ids, const int32_t *__restrict__ owner_req,
    const int32_t *__restrict__ owner_slot, uint32_t *page_tags, int num_pages, int32_t *page_table,
    uint32_t *expected_tags, int batch, int max_pages)
{
    const int k = blockIdx.x * kThreads + threadIdx.x;
    if (k >= n)
        return;
    const int32_t page = page_ids[k];
    if (page < 0 || page >= num_pages)
        return;
    const uint32_t tag = atomicAdd(&page_tags[page], 1u) + 1u;
    if (owner_req == nullptr)
        return;
    const int32_t b = owner_req[k], i = owner_slot[k];
    if (b < 0 || b >= batch || i < 0 || i >= max_pages)
        return;
    const int64_t at = static_cast<int64_t>(b) * max_pages + i;
    expected_tags[at] = tag;
    if (page_table != nullptr)
        page_table[at] = page;
}

}  // namespace

hipError_t launch_tag_check(int batch, int max_pages, int page_size, const int32_t *page_table,
                            const int32_t *context_lens, const uint32_t *expected_tags,
                            const uint32_t *page_tags, int num_pages, int32_t *status,
                            hipStream_t stream)
{
    hipLaunchKernelGGL(tag_check_kernel, dim3(batch), dim3(kThreads), 0, stream, max_pages,
                       page_size, page_table, context_lens, expected_tags, page_tags, num_pages,
                       status);
    return hipGetLastError();
}

hipError_t launch_tag_realloc(int n, const int32_t *page_ids, const int32_t *owner_req,
                              const int32_t *owner_slot, uint32_t *page_tags, int num_pages,
                              int32_t *page_table, uint32_t *expected_tags, int batch,
                              int max_pages, hipStream_t stream)
{
    hipLaunchKernelGGL(tag_realloc_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0,
                       stream, n, page_ids, owner_req, owner_slot, page_tags, num_pages, page_table,
                       expected_tags, batch, max_pages);
    return hipGetLastError();
}

}  // namespace pafp8
