// kv_write.hip -- quantise-on-write into the paged cache, and the codec
// conformance kernels.
//
// Cloudflare, "Smaller, faster, safer: running Kimi and GLM at scale",
// section "KV 缓存量化" (KV cache quantization): decode stores K/V as FP8
// e4m3 instead of BF16 (half the bytes), while prefill keeps BF16.  The same
// encoder serves the decode step's append (one token per request, at
// position context_lens[b] - 1) and the prefill-to-decode hand-off (a block
// of tokens per request); each has its kernel.
//
// Append (one token per request): one work-group per (request, KV head),
// thread d owning head dimension d.  The checked variant first derives the
// request's page-tag verdict (every work-group of the request computes the
// same value) and writes nothing for a request that fails it.
//
// Fill (a block of tokens per request): one work-group per (request, KV head,
// aligned segment of the block layout).  The segment's K and V source rows
// are staged in LDS by coalesced 16-byte loads; K then leaves in the order of
// the block layout (a wave stores 1 KiB of consecutive chunks) and V as
// 16-byte runs of one head dim, read down an LDS column.
#include "pafp8_device.hpp"
#include "pafp8_internal.hpp"
#include "pafp8_quant.hpp"
#include "tag_verify.hpp"

namespace pafp8 {
namespace {

template <bool BF16, int D, bool CHECKED>
__global__ __launch_bounds__(D) void kv_append_kernel(WriteParams p)
{
    const int g = blockIdx.x % p.num_kv_heads;
    const int b = blockIdx.x / p.num_kv_heads;
    const int d = threadIdx.x;
    const int64_t cap = static_cast<int64_t>(p.max_pages) << p.log2_page;

    if constexpr (CHECKED) {
        const int flags = request_flags<D>(b, p.max_pages, 1 << p.log2_page, p.page_table,
                                           p.context_lens, p.expected_tags, p.page_tags, p.num_pages);
        if (g == 0 && d == 0)
            p.status_out[b] = flags;
        if (flags != 0)
            return;
    } else {
        if (p.req_status != nullptr && p.req_status[b] != 0)
            return;
    }
    const int32_t L = p.context_lens[b];
    if (L < 1 || L > cap)
        return;
    const int64_t pos = L - 1;
    const int32_t page = p.page_table[static_cast<int64_t>(b) * p.max_pages + (pos >> p.log2_page)];
    if (page < 0 || page >= p.num_pages)
        return;
    constexpr int E = BF16 ? 2 : 1;
    constexpr int LOG2_TG = BF16 ? 3 : 4, KL = D * E / 64;
    const int slot = static_cast<int>(pos & ((int64_t{1} << p.log2_page) - 1));
    const int64_t head_block = (static_cast<int64_t>(page) * p.num_kv_heads + g) << p.log2_page;
    // Block layout (include/pafp8.h): segments of SEG = min(P, 64/E) slots.
    // K: slot TG*sub + 4j + a of a segment (TG = 16/E) keeps its 16-byte
    // chunk q*KL + l at chunk ((j*KL + l)*4 + q)*(4*NS) + 4*sub + a, NS =
    // SEG/TG; thread d's element is byte (d*E) % 16 of chunk d*E/16.  V: a
    // segment is [D][SEG].
    const int log2_seg = p.log2_page < (BF16 ? 5 : 6) ? p.log2_page : (BF16 ? 5 : 6);
    const int log2_ns = log2_seg - LOG2_TG;
    const int seg = slot >> log2_seg, u = slot & ((1 << log2_seg) - 1);
    const int w = u & ((1 << LOG2_TG) - 1);
    const int c = d * E / 16;
    const int kq = c / KL, kl = c % KL;
    uint8_t *kdst = p.k_pool + (head_block * D + (static_cast<int64_t>(seg) * D << log2_seg)) * E +
                    (((((w >> 2) * KL + kl) * 4 + kq) << (2 + log2_ns)) + ((u >> LOG2_TG) << 2) + (w & 3)) * 16 +
                    (d * E) % 16;
    uint8_t *vdst = p.v_pool + (head_block * D + ((static_cast<int64_t>(seg) * D + d) << log2_seg) + u) * E;
    const int64_t src = (static_cast<int64_t>(b) * p.num_kv_heads + g) * D + d;
    const uint16_t kx = p.k_src[src];
    const uint16_t vx = p.v_src[src];
    if (BF16) {
        *reinterpret_cast<uint16_t *>(kdst) = kx;
        *reinterpret_cast<uint16_t *>(vdst) = vx;
    } else {
        *kdst = static_cast<uint8_t>(quantize_bf16(kx, make_quantizer(p.k_scale[g])));
        *vdst = static_cast<uint8_t>(quantize_bf16(vx, make_quantizer(p.v_scale[g])));
    }
}

constexpr int kFillThreads = 256;

template <bool BF16, int D>
__global__ __launch_bounds__(kFillThreads) void kv_fill_kernel(WriteParams p, int segs_per_req)
{
    constexpr int E = BF16 ? 2 : 1;
    constexpr int LOG2_MAXSEG = BF16 ? 5 : 6;   // 64 bytes per element column
    constexpr int MAXSEG = 1 << LOG2_MAXSEG;
    constexpr int LOG2_TG = BF16 ? 3 : 4;       // tokens per K token group (16 / E)
    constexpr int R = D * E / 16;               // 16-byte chunks per K row
    constexpr int KL = R / 4;
    constexpr int TR = 16 / E;                  // tokens per 16-byte V run
    constexpr int RS = D + 8;                   // LDS row stride (bf16), 16 bytes of padding
    __shared__ __align__(16) uint16_t kt[MAXSEG * RS];
    __shared__ __align__(16) uint16_t vt[MAXSEG * RS];

    const int k = blockIdx.x % segs_per_req;
    const int bg = blockIdx.x / segs_per_req;
    const int g = bg % p.num_kv_heads;
    const int b = bg / p.num_kv_heads;
    const int tid = threadIdx.x;
    if (p.req_status != nullptr && p.req_status[b] != 0)
        return;
    const int T = p.src_tokens;
    const int64_t start = p.token_start[b];
    int64_t count = p.token_count[b];
    if (count > T)
        count = T;
    if (count <= 0)
        return;
    const int log2_seg = p.log2_page < LOG2_MAXSEG ? p.log2_page : LOG2_MAXSEG;
    const int SEG = 1 << log2_seg;
    const int64_t cap = static_cast<int64_t>(p.max_pages) << p.log2_page;
    const int64_t pos0 = ((start >> log2_seg) + k) << log2_seg;  // first position of the segment
    int64_t lo = pos0 > start ? pos0 : start;
    if (lo < 0)
        lo = 0;
    int64_t hi = pos0 + SEG;
    if (hi > start + count)
        hi = start + count;
    if (hi > cap)
        hi = cap;
    if (lo >= hi)
        return;
    const int32_t page = p.page_table[static_cast<int64_t>(b) * p.max_pages + (pos0 >> p.log2_page)];
    if (page < 0 || page >= p.num_pages)
        return;
    const int u_lo = static_cast<int>(lo - pos0), u_hi = static_cast<int>(hi - pos0);
    const int seg = static_cast<int>(pos0 & ((int64_t{1} << p.log2_page) - 1)) >> log2_seg;
    const int64_t seg_elem = (((static_cast<int64_t>(page) * p.num_kv_heads + g) << p.log2_page) +
                              (static_cast<int64_t>(seg) << log2_seg)) * D;
    uint8_t *kseg = p.k_pool + seg_elem * E;
    uint8_t *vseg = p.v_pool + seg_elem * E;

    // stage the segment's source rows (zeros outside [lo, hi)); every load
    // of a thread is issued before the first LDS store
    const int64_t row_stride = static_cast<int64_t>(p.num_kv_heads) * D;
    const int64_t src0 = (static_cast<int64_t>(b) * T * p.num_kv_heads + g) * D;
    constexpr int NLD = (MAXSEG * D / 8 + kFillThreads - 1) / kFillThreads;
    u32x4 kx[NLD], vx[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int idx = tid + i * kFillThreads;
        const int u = idx / (D / 8), c8 = idx % (D / 8);
        kx[i] = vx[i] = u32x4{0u, 0u, 0u, 0u};
        if (u >= u_lo && u < u_hi) {
            const int64_t off = src0 + (pos0 + u - start) * row_stride + c8 * 8;
            kx[i] = load16(p.k_src + off);
            vx[i] = load16(p.v_src + off);
        }
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int idx = tid + i * kFillThreads;
        const int u = idx / (D / 8), c8 = idx % (D / 8);
        if (u < SEG) {
            *reinterpret_cast<u32x4 *>(&kt[u * RS + c8 * 8]) = kx[i];
            *reinterpret_cast<u32x4 *>(&vt[u * RS + c8 * 8]) = vx[i];
        }
    }
    __syncthreads();

    const E4m3Quantizer ks = make_quantizer(BF16 ? 1.0f : p.k_scale[g]);
    const E4m3Quantizer vs = make_quantizer(BF16 ? 1.0f : p.v_scale[g]);
    // K: this thread's chunk positions cp, in storage order; chunk cp holds
    // chunk c = q*KL + l of slot u = TG*s + 4j + a
    const int log2_ns = log2_seg - LOG2_TG;
    constexpr int NK = (MAXSEG * R + kFillThreads - 1) / kFillThreads;
#pragma unroll
    for (int it = 0; it < NK; ++it) {
        const int cp = tid + it * kFillThreads;
        if (cp >= SEG * R)
            break;
        const int a = cp & 3;
        const int s_ = (cp >> 2) & ((1 << log2_ns) - 1);
        const int rest = cp >> (2 + log2_ns);
        const int q = rest & 3, jl = rest >> 2;
        const int j = jl / KL, l = jl % KL;
        const int u = (s_ << LOG2_TG) + 4 * j + a;
        if (u < u_lo || u >= u_hi)
            continue;
        const uint16_t *row = &kt[u * RS + (q * KL + l) * (16 / E)];
        u32x4 out;
        if (BF16) {
            out = *reinterpret_cast<const u32x4 *>(row);
        } else {
            const u32x4 x0 = *reinterpret_cast<const u32x4 *>(row);
            const u32x4 x1 = *reinterpret_cast<const u32x4 *>(row + 8);
            out = u32x4{quantize_bf16x4(x0[0], x0[1], ks), quantize_bf16x4(x0[2], x0[3], ks),
                        quantize_bf16x4(x1[0], x1[1], ks), quantize_bf16x4(x1[2], x1[3], ks)};
        }
        store16(kseg + cp * 16, out);
    }
    // V: runs of TR slots of one head dim, the dim fastest across lanes
    constexpr int NV = (MAXSEG / TR * D + kFillThreads - 1) / kFillThreads;
#pragma unroll
    for (int it = 0; it < NV; ++it) {
        const int idx = tid + it * kFillThreads;
        if (idx >= (SEG / TR) * D)
            break;
        const int d = idx % D, r = idx / D;
        const int u0 = r * TR;
        uint32_t word[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int u = u0 + e * (TR / 4);
            if (BF16) {
                word[e] = static_cast<uint32_t>(vt[u * RS + d]) | static_cast<uint32_t>(vt[(u + 1) * RS + d]) << 16;
            } else {
                word[e] = quantize_bf16x4(static_cast<uint32_t>(vt[u * RS + d]) | static_cast<uint32_t>(vt[(u + 1) * RS + d]) << 16,
                                    static_cast<uint32_t>(vt[(u + 2) * RS + d]) | static_cast<uint32_t>(vt[(u + 3) * RS + d]) << 16,
                                    vs);
            }
        }
        uint8_t *dst = vseg + (static_cast<int64_t>(d) * SEG + u0) * E;
        if (u0 >= u_lo && u0 + TR <= u_hi) {
            store16(dst, u32x4{word[0], word[1], word[2], word[3]});
        } else {
            for (int t = 0; t < TR; ++t) {
                const int u = u0 + t;
                if (u < u_lo || u >= u_hi)
                    continue;
                if (BF16)
                    reinterpret_cast<uint16_t *>(dst)[t] = static_cast<uint16_t>(word[t >> 1] >> (16 * (t & 1)));
                else
                    dst[t] = static_cast<uint8_t>(word[t >> 2] >> (8 * (t & 3)));
            }
        }
    }
}

template <bool BF16, int D>
hipError_t launch_write_t(const WriteParams &p, hipStream_t stream)
{
    if (p.context_lens != nullptr) {
        const int64_t blocks = static_cast<int64_t>(p.batch) * p.num_kv_heads;
        if (blocks > 0x7FFFFFFF)
            return hipErrorInvalidConfiguration;
        if (p.status_out != nullptr)
            hipLaunchKernelGGL((kv_append_kernel<BF16, D, true>), dim3(static_cast<unsigned>(blocks)),
                               dim3(D), 0, stream, p);
        else
            hipLaunchKernelGGL((kv_append_kernel<BF16, D, false>), dim3(static_cast<unsigned>(blocks)),
                               dim3(D), 0, stream, p);
        return hipGetLastError();
    }
    const int log2_maxseg = BF16 ? 5 : 6;
    const int log2_seg = p.log2_page < log2_maxseg ? p.log2_page : log2_maxseg;
    // segments one request's span can touch: ceil(T / SEG) + 1 (an unaligned start)
    const int segs = ((p.src_tokens + (1 << log2_seg) - 1) >> log2_seg) + 1;
    const int64_t blocks = static_cast<int64_t>(p.batch) * p.num_kv_heads * segs;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((kv_fill_kernel<BF16, D>), dim3(static_cast<unsigned>(blocks)), dim3(kFillThreads),
                       0, stream, p, segs);
    return hipGetLastError();
}

// --- codec conformance kernels -------------------------------------------------

// four values per thread through the packed encoder the fill kernel uses, so
// the exhaustive sweep covers every byte position of it
__global__ __launch_bounds__(256) void e4m3_encode_kernel(const float *__restrict__ x,
                                                          uint8_t *__restrict__ codes, int64_t n)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int64_t n4 = (n + 3) / 4;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const int64_t e = 4 * i;
        if (e + 4 <= n) {
            const uint32_t w = e4m3_encode4(x[e], x[e + 1], x[e + 2], x[e + 3]);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                codes[e + k] = static_cast<uint8_t>(w >> (8 * k));
        } else {
            for (int64_t k = e; k < n; ++k)
                codes[k] = static_cast<uint8_t>(e4m3_encode(x[k]));
        }
    }
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
    int64_t blocks = (n + 1023) / 1024;
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
