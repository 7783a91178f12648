// tag_check.hip -- the batched page-tag integrity check.
//
// Cloudflare, "Smaller, faster, safer: running Kimi and GLM at scale",
// section "共享 KV 缓存保护" (shared KV cache protection): each physical page
// carries a tag that changes when the page is reallocated; the server keeps,
// per request, the pages and tags it expects, and verifies them before decode
// reads the cache; a mismatch terminates that request.  The post runs the
// verification as its own batched pass rather than inside the attention
// kernel (fusing it would race between GPU thread groups); this kernel is
// that pass: one work-group per request, stream-ordered before append and
// attention, which read its per-request verdict.
#include "pafp8_device.hpp"
#include "pafp8_internal.hpp"

namespace pafp8 {
namespace {

constexpr int kTagMismatch = 1;
constexpr int kPageOob = 2;
constexpr int kBadLen = 4;
constexpr int kThreads = 256;
constexpr int kChunk = 16;  // page-table entries per thread per pass

__global__ __launch_bounds__(kThreads) void tag_check_kernel(
    int max_pages, int page_size, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ context_lens, const uint32_t *__restrict__ expected_tags,
    const uint32_t *__restrict__ page_tags, int num_pages, int32_t *__restrict__ status)
{
    const int b = blockIdx.x;
    const int32_t L = context_lens[b];
    const bool bad_len = L < 1 || static_cast<int64_t>(L) > static_cast<int64_t>(max_pages) * page_size;
    int flags = 0;
    if (!bad_len) {
        const int n = static_cast<int>((static_cast<int64_t>(L) + page_size - 1) / page_size);
        const int32_t *row = page_table + static_cast<int64_t>(b) * max_pages;
        const uint32_t *exp_row = expected_tags + static_cast<int64_t>(b) * max_pages;
        // kChunk entries per thread per pass, every load issued before any
        // compare: a long request costs two memory round trips per pass
        // instead of two per 256 entries.  Indices past n read entry n - 1
        // again (n >= 1) and are not judged.
        for (int base = 0; base < n; base += kThreads * kChunk) {
            int32_t page[kChunk];
            uint32_t want[kChunk], have[kChunk];
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                const int i = min(base + j * kThreads + static_cast<int>(threadIdx.x), n - 1);
                page[j] = row[i];
                want[j] = exp_row[i];
            }
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                const bool in_pool = page[j] >= 0 && page[j] < num_pages;
                have[j] = in_pool ? page_tags[page[j]] : 0u;  // the pool may be empty
            }
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                if (base + j * kThreads + static_cast<int>(threadIdx.x) >= n)
                    continue;
                if (page[j] < 0 || page[j] >= num_pages)
                    flags |= kPageOob;
                else if (have[j] != want[j])
                    flags |= kTagMismatch;
            }
        }
    }
    const int any_tag = __syncthreads_or(flags & kTagMismatch);
    const int any_oob = __syncthreads_or(flags & kPageOob);
    if (threadIdx.x == 0)
        status[b] = bad_len ? kBadLen : ((any_tag ? kTagMismatch : 0) | (any_oob ? kPageOob : 0));
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

}  // namespace pafp8
