// pafp8_internal.hpp -- launchers shared between the C-ABI layer and the
// kernel translation units.  Host-side validation happens in api.hip before
// any of these is called; they assume their arguments are consistent.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "attn_params.hpp"

namespace pafp8 {

hipError_t launch_splitk_combine(const float *part_o, const float *part_lse, int batch,
                                 int num_q_heads, int num_splits, int head_dim,
                                 const int32_t *req_status, float *out, float *lse,
                                 hipStream_t stream);

// merge of a balanced attention launch's partials (W = groups work-groups
// per KV head; prefix = the [B + 1] array the attention kernel stored)
hipError_t launch_bal_combine(const float *part_o, const float *part_lse, const int64_t *prefix,
                              int batch, int num_q_heads, int groups, int head_dim,
                              const int32_t *req_status, const int32_t *context_lens,
                              int max_pages, int log2_page, float *out, float *lse,
                              hipStream_t stream);

hipError_t launch_tag_realloc(int n, const int32_t *page_ids, const int32_t *owner_req,
                              const int32_t *owner_slot, uint32_t *page_tags, int num_pages,
                              int32_t *page_table, uint32_t *expected_tags, int batch,
                              int max_pages, hipStream_t stream);

hipError_t launch_tag_check(int batch, int max_pages, int page_size, const int32_t *page_table,
                            const int32_t *context_lens, const uint32_t *expected_tags,
                            const uint32_t *page_tags, int num_pages, int32_t *status,
                            hipStream_t stream);

// Quantise-on-write.  append mode (context_lens != nullptr): one token per
// request at context_lens[b] - 1 from src [B][1][Hkv][D]; fill mode: tokens
// token_start[b] + j, j < min(token_count[b], src_tokens), from
// src [B][src_tokens][Hkv][D].
struct WriteParams {
    uint8_t *k_pool;
    uint8_t *v_pool;
    const float *k_scale;
    const float *v_scale;
    const int32_t *page_table;
    const int32_t *req_status;    // nullable
    const int32_t *context_lens;  // append mode
    const int32_t *token_start;   // fill mode
    const int32_t *token_count;   // fill mode
    const uint16_t *k_src;
    const uint16_t *v_src;
    int32_t src_tokens;
    int32_t num_pages;
    int32_t log2_page;
    int32_t num_kv_heads;
    int32_t batch;
    int32_t max_pages;
    // append with the tag check fused (status_out != nullptr): the verdict of
    // page_tag_check is computed per request, written to status_out, and a
    // non-zero verdict skips the write; req_status is then not read
    const uint32_t *page_tags;
    const uint32_t *expected_tags;
    int32_t *status_out;
};

hipError_t launch_kv_write(bool bf16_pool, int head_dim, const WriteParams &p,
                           hipStream_t stream);

// INT4 weight streaming: y[M][N] = x[M][K] . (q * s)^T, w in packed blocks.
hipError_t launch_int4_gemv(const uint16_t *x, int M, const uint8_t *w, const uint16_t *scales,
                            int N, int K, float *y, int num_cus, hipStream_t stream);
hipError_t launch_int4_pack(const uint8_t *src, uint8_t *dst, int N, int K, hipStream_t stream);

// Measurement: a bare read of bytes (a multiple of kStreamReadTile) by
// work_groups work-groups of 256 threads; sink holds work_groups * 256 words.
constexpr int64_t kStreamReadTile = 16384;
constexpr int kStreamReadThreads = 256;
hipError_t launch_stream_read(const void *src, int64_t bytes, int work_groups, uint32_t *sink,
                              hipStream_t stream);
// ... and write src_bytes / ratio bytes to dst (ratio 1, 2 or 4)
hipError_t launch_stream_read_write(const void *src, int64_t src_bytes, void *dst, int ratio,
                                    int work_groups, hipStream_t stream);

hipError_t launch_e4m3_encode(const float *x, uint8_t *codes, int64_t n, hipStream_t stream);
hipError_t launch_e4m3_decode(const uint8_t *codes, float *f32, float *via_f16, float *via_bf16,
                              int64_t n, hipStream_t stream);

}  // namespace pafp8
