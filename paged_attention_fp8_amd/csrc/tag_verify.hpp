// tag_verify.hpp -- the per-request page-tag verdict, shared by the batched
// check pass and the append kernel that fuses it.
//
// Cloudflare, "Smaller, faster, safer: running Kimi and GLM at scale",
// section "共享 KV 缓存保护" (shared KV cache protection): a request may read
// its pages only if every page still carries the tag the request recorded
// when the page was given to it.  Every thread of a work-group calls
// request_flags for the same request and gets the same verdict: the OR of
// PAGE_OOB / TAG_MISMATCH over its pages, or BAD_LEN alone.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pafp8 {

constexpr int kTagMismatch = 1;
constexpr int kPageOob = 2;
constexpr int kBadLen = 4;

// NT threads per work-group; each issues kChunk page-table and expected-tag
// loads, then kChunk tag gathers, before comparing, so a pass over
// NT * kChunk pages costs two memory round trips.
template <int NT>
__device__ __forceinline__ int request_flags(int b, int max_pages, int page_size,
                                             const int32_t *__restrict__ page_table,
                                             const int32_t *__restrict__ context_lens,
                                             const uint32_t *__restrict__ expected_tags,
                                             const uint32_t *__restrict__ page_tags, int num_pages)
{
    constexpr int kChunk = 16;
    const int tid = static_cast<int>(threadIdx.x);
    const int32_t L = context_lens[b];
    const bool bad_len = L < 1 || static_cast<int64_t>(L) > static_cast<int64_t>(max_pages) * page_size;
    int flags = 0;
    if (!bad_len) {
        const int n = static_cast<int>((static_cast<int64_t>(L) + page_size - 1) / page_size);
        const int32_t *row = page_table + static_cast<int64_t>(b) * max_pages;
        const uint32_t *exp_row = expected_tags + static_cast<int64_t>(b) * max_pages;
        // indices past n read entry n - 1 again (n >= 1) and are not judged
        for (int base = 0; base < n; base += NT * kChunk) {
            int32_t page[kChunk];
            uint32_t want[kChunk], have[kChunk];
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                const int i = min(base + j * NT + tid, n - 1);
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
                if (base + j * NT + tid >= n)
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
    return bad_len ? kBadLen : ((any_tag ? kTagMismatch : 0) | (any_oob ? kPageOob : 0));
}

}  // namespace pafp8
