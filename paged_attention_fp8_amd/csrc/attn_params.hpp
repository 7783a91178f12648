// attn_params.hpp -- the decode attention launch: its parameter block and
// launcher, shared by decode_attn.hip and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pafp8 {

// Decode attention over one batch (both pool types).
struct AttnParams {
    const uint8_t *k_pool;
    const uint8_t *v_pool;
    const float *k_scale;  // nullptr for bf16 pools
    const float *v_scale;
    const int32_t *page_table;
    const int32_t *context_lens;
    const int32_t *req_status;  // nullable
    const uint16_t *q;
    const uint16_t *k_new;  // this step's token [B][Hkv][D] when the launch also appends it, else nullptr
    const uint16_t *v_new;
    float *out;        // final [B][Hq][D] (when S == 1, and whole requests of a balanced launch)
    float *lse;        // final [B][Hq] or nullptr
    float *part_o;     // [B][Hq][S][D] (when S > 1); balanced: [Hq][B + W - 1][D]
    float *part_lse;   // [B][Hq][S]; balanced: [Hq][B + W - 1]
    int64_t *bal_prefix;  // balanced: [B + 1] first page of each request in the sequence, then C
    int32_t num_pages;
    int32_t log2_page;  // page_size = 1 << log2_page
    int32_t num_kv_heads;
    int32_t batch;
    int32_t max_pages;
    int32_t num_q_heads;
    int32_t group;            // num_q_heads / num_kv_heads
    int32_t num_splits;       // S (1 in a balanced launch)
    int32_t pages_per_split;  // ceil(max_pages / S)
    int32_t wave_parts;       // > 0: wave-per-split mode, each wave takes this many splits
    int32_t part_tiles;       // wave mode: tiles in one split
    int32_t bal_groups;       // W work-groups per KV head in a balanced launch, else 0
    float sm_scale;
};

hipError_t launch_decode_attn(bool bf16_pool, int head_dim, const AttnParams &p,
                              hipStream_t stream);

}  // namespace pafp8
