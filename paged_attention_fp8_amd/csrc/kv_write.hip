// kv_write.hip -- quantise-on-write into the paged cache, and the codec
// conformance kernels.
//
// Cloudflare, "Smaller, faster, safer: running Kimi and GLM at scale",
// section "KV 缓存量化" (KV cache quantization): decode stores K/V as FP8
// e4m3 instead of BF16 (half the bytes), while prefill keeps BF16.  The same
// kernel serves the decode step's append (one token per request, at position
// context_lens[b] - 1) and the prefill-to-decode hand-off (a block of tokens
// per request).
//
// Work split: one work-group per (request, KV head, 16 consecutive positions).
// Positions are grouped on 16-aligned boundaries so that a group never spans
// two pages (pages hold a multiple of 16 tokens).  Thread d owns one head
// dimension: its K codes land in the 16-byte chunks of the block layout
// (consecutive threads fill a chunk), its V codes form one contiguous run of
// 16 slots of a V row and leave as a single 16-byte store (two for bf16).
#include "pafp8_device.hpp"
#include "pafp8_internal.hpp"

namespace pafp8 {
namespace {

template <bool BF16, int D>
__global__ __launch_bounds__(D) void kv_write_kernel(WriteParams p, int groups_per_req)
{
    const int k = blockIdx.x % groups_per_req;
    const int bg = blockIdx.x / groups_per_req;
    const int g = bg % p.num_kv_heads;
    const int b = bg / p.num_kv_heads;
    const int d = threadIdx.x;
    const int P = 1 << p.log2_page;
    const int64_t cap = static_cast<int64_t>(p.max_pages) << p.log2_page;

    if (p.req_status != nullptr && p.req_status[b] != 0)
        return;
    int64_t start, count;
    int T;
    if (p.context_lens != nullptr) {
        const int32_t L = p.context_lens[b];
        if (L < 1 || L > cap)
            return;
        start = L - 1;
        count = 1;
        T = 1;
    } else {
        T = p.src_tokens;
        start = p.token_start[b];
        count = p.token_count[b];
        if (count > T)
            count = T;
        if (count <= 0)
            return;
    }
    const int64_t g0 = ((start >> 4) + k) << 4;
    int64_t lo = g0 > start ? g0 : start;
    if (lo < 0)
        lo = 0;
    int64_t hi = g0 + 16;
    if (hi > start + count)
        hi = start + count;
    if (hi > cap)
        hi = cap;
    if (lo >= hi)
        return;

    const int32_t page = p.page_table[static_cast<int64_t>(b) * p.max_pages + (g0 >> p.log2_page)];
    if (page < 0 || page >= p.num_pages)
        return;
    const int slot0 = static_cast<int>(g0 & (P - 1));
    constexpr int E = BF16 ? 2 : 1;
    const int64_t head_block = (static_cast<int64_t>(page) * p.num_kv_heads + g) * P * D;
    // Block layout (include/pafp8.h): segments of SEG = min(P, 64/E) tokens.
    // K: token TG*sub + 4j + a of a segment (TG = 16/E) keeps its 16-byte
    // chunk q*KL + l at chunk ((j*KL + l)*4 + q)*(4*NS) + 4*sub + a, NS =
    // SEG/TG; thread d's element is byte (d*E) % 16 of chunk d*E/16.  V: a
    // segment is [D][SEG]; the 16 aligned positions of this work-group lie in
    // one segment, so thread d's 16 V codes are contiguous.
    constexpr int LOG2_TG = BF16 ? 3 : 4, KL = D * E / 64;
    const int log2_seg = p.log2_page < (BF16 ? 5 : 6) ? p.log2_page : (BF16 ? 5 : 6);
    const int log2_ns = log2_seg - LOG2_TG;
    const int c = d * E / 16;
    const int kq = c / KL, kl = c % KL;
    uint8_t *kblock = p.k_pool + head_block * E + (d * E) % 16;
    const int seg0 = slot0 >> log2_seg, u0 = slot0 & ((1 << log2_seg) - 1);
    uint8_t *vdst = p.v_pool + (head_block + ((static_cast<int64_t>(seg0) * D + d) << log2_seg) + u0) * E;
    const float ks = BF16 ? 1.0f : p.k_scale[g];
    const float vs = BF16 ? 1.0f : p.v_scale[g];
    const int64_t src_stride = static_cast<int64_t>(p.num_kv_heads) * D;  // per token
    const uint16_t *ksrc = p.k_src + (static_cast<int64_t>(b) * T * p.num_kv_heads + g) * D + d;
    const uint16_t *vsrc = p.v_src + (static_cast<int64_t>(b) * T * p.num_kv_heads + g) * D + d;

    constexpr int NV = BF16 ? 8 : 4;  // dwords holding the 16 V slots
    uint32_t vword[NV] = {};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t pos = g0 + i;
        if (pos < lo || pos >= hi)
            continue;
        const int64_t j = pos - start;
        const uint16_t kx = ksrc[j * src_stride];
        const uint16_t vx = vsrc[j * src_stride];
        // token i of this 16-position group: segment-relative token u
        const int u = u0 + i;
        const int w = u & ((1 << LOG2_TG) - 1);
        uint8_t *kdst = kblock + seg0 * ((D * E) << log2_seg) +
                        (((((w >> 2) * KL + kl) * 4 + kq) << (2 + log2_ns)) + ((u >> LOG2_TG) << 2) + (w & 3)) * 16;
        if (BF16) {
            *reinterpret_cast<uint16_t *>(kdst) = kx;
            vword[i >> 1] |= static_cast<uint32_t>(vx) << (16 * (i & 1));
        } else {
            *kdst = static_cast<uint8_t>(quantize_bf16(kx, ks));
            vword[i >> 2] |= quantize_bf16(vx, vs) << (8 * (i & 3));
        }
    }
    if (lo == g0 && hi == g0 + 16) {
#pragma unroll
        for (int w = 0; w < NV; w += 4)
            store16(vdst + 4 * w, u32x4{vword[w], vword[w + 1], vword[w + 2], vword[w + 3]});
    } else {
        for (int i = static_cast<int>(lo - g0); i < static_cast<int>(hi - g0); ++i) {
            if (BF16)
                reinterpret_cast<uint16_t *>(vdst)[i] = static_cast<uint16_t>(vword[i >> 1] >> (16 * (i & 1)));
            else
                vdst[i] = static_cast<uint8_t>(vword[i >> 2] >> (8 * (i & 3)));
        }
    }
}

template <bool BF16, int D>
hipError_t launch_write_t(const WriteParams &p, hipStream_t stream)
{
    const int groups = p.context_lens != nullptr ? 1 : (p.src_tokens + 15) / 16 + 1;
    const int64_t blocks = static_cast<int64_t>(p.batch) * p.num_kv_heads * groups;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((kv_write_kernel<BF16, D>), dim3(static_cast<unsigned>(blocks)), dim3(D), 0,
                       stream, p, groups);
    return hipGetLastError();
}

// --- codec conformance kernels -------------------------------------------------

__global__ __launch_bounds__(256) void e4m3_encode_kernel(const float *__restrict__ x,
                                                          uint8_t *__restrict__ codes, int64_t n)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        codes[i] = static_cast<uint8_t>(e4m3_encode(x[i]));
}

__global__ __launch_bounds__(256) void e4m3_decode_kernel(const uint8_t *__restrict__ codes,
                                                          float *f32, float *via_f16,
                                                          float *via_bf16, int64_t n)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint32_t w = codes[i];
        if (f32)
            f32[i] = e4m3x2_to_f32x2<false>(w)[0];
        if (via_f16) {
            const u32x2 h = e4m3x4_to_f16x4(w);
            via_f16[i] = static_cast<float>(__builtin_bit_cast(f16x2, h[0])[0]);
        }
        if (via_bf16) {
            const u32x2 h = e4m3x4_to_bf16x4(w);
            via_bf16[i] = bf16_lo(h[0]);
        }
    }
}

unsigned grid_for(int64_t n)
{
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    return static_cast<unsigned>(blocks < 1 ? 1 : blocks);
}

}  // namespace

hipError_t launch_kv_write(bool bf16_pool, int head_dim, const WriteParams &p,
                           hipStream_t stream)
{
    if (bf16_pool)
        return head_dim == 64 ? launch_write_t<true, 64>(p, stream) : launch_write_t<true, 128>(p, stream);
    return head_dim == 64 ? launch_write_t<false, 64>(p, stream) : launch_write_t<false, 128>(p, stream);
}

hipError_t launch_e4m3_encode(const float *x, uint8_t *codes, int64_t n, hipStream_t stream)
{
    hipLaunchKernelGGL(e4m3_encode_kernel, dim3(grid_for(n)), dim3(256), 0, stream, x, codes, n);
    return hipGetLastError();
}

hipError_t launch_e4m3_decode(const uint8_t *codes, float *f32, float *via_f16, float *via_bf16,
                              int64_t n, hipStream_t stream)
{
    hipLaunchKernelGGL(e4m3_decode_kernel, dim3(grid_for(n)), dim3(256), 0, stream, codes, f32,
                       via_f16, via_bf16, n);
    return hipGetLastError();
}

}  // namespace pafp8
