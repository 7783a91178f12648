// pafp8_append.hpp -- one element of a decode step's new token written into
// the paged cache: the append kernel and the attention kernels that take the
// append into their own launch share it.
//
// Cloudflare, "Smaller, faster, safer: running Kimi and GLM at scale",
// section "KV 缓存量化" (KV cache quantization): decode stores K/V as FP8
// e4m3 (bf16 pools keep the bits).
#pragma once

#include "pafp8_quant.hpp"

namespace pafp8 {

// Head dim d of KV head g of the token in slot `slot` of physical page `page`
// (page inside the pool).  Block layout (include/pafp8.h): segments of
// SEG = min(P, 64/E) slots.  K: slot TG*sub + 4j + a of a segment (TG = 16/E)
// keeps its 16-byte chunk q*KL + l at chunk ((j*KL + l)*4 + q)*(4*NS) + 4*sub + a,
// NS = SEG/TG; element d is byte (d*E) % 16 of chunk d*E/16.  V: a segment
// is [D][SEG].  NT: non-temporal stores (used when the append runs inside the
// attention launch, where the token's scattered V bytes are written while
// every other work-group streams the pool).
template <bool BF16, int D, bool NT = false>
__device__ __forceinline__ void append_token_element(uint8_t *k_pool, uint8_t *v_pool, int32_t page,
                                                     int num_kv_heads, int g, int log2_page, int slot,
                                                     int d, uint16_t kx, uint16_t vx, float k_scale,
                                                     float v_scale)
{
    constexpr int E = BF16 ? 2 : 1;
    constexpr int LOG2_TG = BF16 ? 3 : 4, KL = D * E / 64;
    const int64_t head_block = (static_cast<int64_t>(page) * num_kv_heads + g) << log2_page;
    const int log2_seg = log2_page < (BF16 ? 5 : 6) ? log2_page : (BF16 ? 5 : 6);
    const int log2_ns = log2_seg - LOG2_TG;
    const int seg = slot >> log2_seg, u = slot & ((1 << log2_seg) - 1);
    const int w = u & ((1 << LOG2_TG) - 1);
    const int c = d * E / 16;
    const int kq = c / KL, kl = c % KL;
    uint8_t *kdst = k_pool + (head_block * D + (static_cast<int64_t>(seg) * D << log2_seg)) * E +
                    (((((w >> 2) * KL + kl) * 4 + kq) << (2 + log2_ns)) + ((u >> LOG2_TG) << 2) + (w & 3)) * 16 +
                    (d * E) % 16;
    uint8_t *vdst = v_pool + (head_block * D + ((static_cast<int64_t>(seg) * D + d) << log2_seg) + u) * E;
    if constexpr (BF16) {
        if constexpr (NT) {
            __builtin_nontemporal_store(kx, reinterpret_cast<uint16_t *>(kdst));
            __builtin_nontemporal_store(vx, reinterpret_cast<uint16_t *>(vdst));
        } else {
            *reinterpret_cast<uint16_t *>(kdst) = kx;
            *reinterpret_cast<uint16_t *>(vdst) = vx;
        }
    } else {
        const uint8_t kc = static_cast<uint8_t>(quantize_bf16(kx, make_quantizer(k_scale)));
        const uint8_t vc = static_cast<uint8_t>(quantize_bf16(vx, make_quantizer(v_scale)));
        if constexpr (NT) {
            __builtin_nontemporal_store(kc, kdst);
            __builtin_nontemporal_store(vc, vdst);
        } else {
            *kdst = kc;
            *vdst = vc;
        }
    }
}

}  // namespace pafp8
