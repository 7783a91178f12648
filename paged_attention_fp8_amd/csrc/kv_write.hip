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
// Fill (a block of tokens per request): work-groups per (request, aligned
// 64-position tile, KV head) and pool.  K rows are quantised in registers and
// stored as 8-byte halves of their chunks; V is transposed by pairing the
// quantised values of one head dim across tokens in the packed conversion,
// and in a whole e4m3 tile of a page of 64 tokens or more its rows are
// assembled in LDS so that they leave as 1 KiB runs.
#include "pafp8_append.hpp"
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
    const int slot = static_cast<int>(pos & ((int64_t{1} << p.log2_page) - 1));
    const int64_t src = (static_cast<int64_t>(b) * p.num_kv_heads + g) * D + d;
    append_token_element<BF16, D>(p.k_pool, p.v_pool, page, p.num_kv_heads, g, p.log2_page, slot, d,
                                  p.k_src[src], p.v_src[src], BF16 ? 1.0f : p.k_scale[g],
                                  BF16 ? 1.0f : p.v_scale[g]);
}

// --- fill ---------------------------------------------------------------------
// Work-groups of four waves, one per (request, 64-position tile, KV head) and
// pool: the first half of the grid writes K, the second half V (the two
// streams run one after the other rather than side by side, which measured
// faster), and the tile index runs fastest.  Wave w handles the tile's
// 16-position group w.  A group lies in one page and one segment (the tile is
// aligned to 64 positions, page_size and SEG are multiples of 16), so each
// wave works on one uniform source base and one uniform segment base,
// addressed through buffer descriptors with 32-bit lane offsets.  Stores that
// must not happen (a page outside the pool, positions outside [lo, hi)) get
// an offset past the descriptor's range, which the hardware drops, so
// nothing branches between a wave's loads and its stores.
//   K wave: a lane owns one 16-byte source piece (8 elements) of the rows
//   lane / (D/8) + i * (512/D); each load instruction reads whole rows and
//   each store lands in runs of four consecutive chunks.
//   V wave: a lane owns D/64 head dims of the group's 16 tokens and pairs the
//   quantised values by token, so each dim leaves as one 16-token run of the
//   [D][SEG] segment.
constexpr int kFillTile = 64;
constexpr int kFillWaves = 4;
constexpr uint32_t kNoWrite = 0x80000000u;   // at or past every descriptor's range
constexpr int kStreamLoad = 2;                // buffer load policy: non-temporal (the source is read once)
constexpr int kFillLdsRow = 80;               // bytes per head dim of the V tile in LDS

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_at(const void *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 0x7FFFFFFF, 0x00020000);
}

struct FillGroup {
    int64_t pos;          // first of the group's 16 positions
    int64_t lo, hi;       // positions written: [lo, hi)
    const char *src;      // source row of position pos (may precede row 0 when pos < lo)
    uint8_t *seg;         // pool segment holding the group
    int row_bytes;        // source bytes per token
    int u0;               // slot of pos within its segment
    int grp;              // group index within the tile (the wave index)
    int log2_seg;
    bool ok;              // the group's page lies inside the pool
};

__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// byte offset in the source of row pos + v, clamped into [lo, hi) (partial groups)
__device__ __forceinline__ uint32_t fill_src_row(const FillGroup &f, int v)
{
    int64_t row = f.pos + v;
    row = row < f.lo ? f.lo : (row >= f.hi ? f.hi - 1 : row);
    return static_cast<uint32_t>(static_cast<int>(row - f.pos) * f.row_bytes);
}

template <bool BF16, int D, bool FAST, bool WHOLE>
__device__ __forceinline__ void fill_k_group(const FillGroup &f, float scale, int lane)
{
    constexpr int E = BF16 ? 2 : 1;
    constexpr int LPR = D / 8;                  // lanes per row: 16-byte source pieces
    constexpr int RPI = 64 / LPR;               // rows per load instruction
    constexpr int NI = 16 / RPI;                // load instructions per group
    constexpr int LOG2_TG = BF16 ? 3 : 4;       // tokens per K token group
    constexpr int KL = D * E / 64;
    const int pc = lane % LPR, rr = lane / LPR;
    const int c = BF16 ? pc : pc >> 1, h = BF16 ? 0 : pc & 1;
    const int q = c / KL, l = c % KL;
    const int log2_ns = f.log2_seg - LOG2_TG;
    const auto src = buffer_at(f.src);
    const auto dst = buffer_at(f.seg);

    u32x4 x[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        if (WHOLE)
            x[i] = __builtin_amdgcn_raw_buffer_load_b128(src, rr * f.row_bytes + pc * 16, i * RPI * f.row_bytes, kStreamLoad);
        else
            x[i] = __builtin_amdgcn_raw_buffer_load_b128(src, fill_src_row(f, i * RPI + rr) + pc * 16, 0, kStreamLoad);
    }
    u32x2 w[NI];
    if (!BF16) {
        const E4m3Quantizer qz = make_quantizer(scale);
        uint64_t nan = 0;
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float f0 = lo_f(x[i][2 * e]), f1 = hi_f(x[i][2 * e]);
                const float f2 = lo_f(x[i][2 * e + 1]), f3 = hi_f(x[i][2 * e + 1]);
                nan |= __builtin_amdgcn_ballot_w64(__builtin_isunordered(f0, f1));
                nan |= __builtin_amdgcn_ballot_w64(__builtin_isunordered(f2, f3));
                const uint32_t v = e4m3_pack2<false>(quotient<FAST>(f0, qz), quotient<FAST>(f1, qz), 0u);
                w[i][e] = e4m3_pack2<true>(quotient<FAST>(f2, qz), quotient<FAST>(f3, qz), v);
            }
        if (nan != 0) {
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    uint32_t v = w[i][e];
                    v = e4m3_patch_nan(v, 0, lo_f(x[i][2 * e]));
                    v = e4m3_patch_nan(v, 1, hi_f(x[i][2 * e]));
                    v = e4m3_patch_nan(v, 2, lo_f(x[i][2 * e + 1]));
                    w[i][e] = e4m3_patch_nan(v, 3, hi_f(x[i][2 * e + 1]));
                }
        }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        // row u = TG*s + 4*j + a of the segment keeps chunk c = q*KL + l at
        // chunk ((j*KL + l)*4 + q) * (4*NS) + 4*s + a, NS = SEG / TG
        const int v = i * RPI + rr;
        const int u = f.u0 + v;
        const int s = u >> LOG2_TG, j = (u >> 2) & ((1 << (LOG2_TG - 2)) - 1), a = u & 3;
        uint32_t off = static_cast<uint32_t>((((((j * KL + l) * 4 + q) << (2 + log2_ns)) + 4 * s + a) * 16) + h * 8);
        bool keep = f.ok;
        if (!WHOLE)
            keep = keep && f.pos + v >= f.lo && f.pos + v < f.hi;
        off = keep ? off : kNoWrite;
        if (BF16)
            __builtin_amdgcn_raw_buffer_store_b128(x[i], dst, off, 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b64(w[i], dst, off, 0, 0);
    }
}

template <bool BF16, int D, bool FAST, bool WHOLE, bool TILE>
__device__ __forceinline__ void fill_v_group(const FillGroup &f, float scale, int lane, uint8_t *lds)
{
    constexpr int DPL = D / 64;                 // head dims per lane: 2 or 1
    const int d0 = lane * DPL;
    const auto src = buffer_at(f.src);
    const auto dst = buffer_at(f.seg);
    const int seg_len = 1 << f.log2_seg;

    // x[t]: dim d0 of token t in the low half, dim d0 + 1 in the high half;
    // the clamped row of a partial group depends on t alone
    uint32_t x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const uint32_t voff = static_cast<uint32_t>(d0 * 2);
        const uint32_t soff = WHOLE ? static_cast<uint32_t>(t * f.row_bytes) : fill_src_row(f, t);
        if (DPL == 2)
            x[t] = __builtin_amdgcn_raw_buffer_load_b32(src, voff, soff, kStreamLoad);
        else
            x[t] = __builtin_amdgcn_raw_buffer_load_b16(src, voff, soff, kStreamLoad);
    }
    if (BF16) {
        // a dword of the run holds tokens 2m (low half) and 2m + 1
#pragma unroll
        for (int k = 0; k < DPL; ++k) {
            const uint32_t sel = k ? 0x07060302u : 0x05040100u;
            uint32_t r[8];
#pragma unroll
            for (int m = 0; m < 8; ++m)
                r[m] = __builtin_amdgcn_perm(x[2 * m + 1], x[2 * m], sel);
            const uint32_t base = static_cast<uint32_t>(((d0 + k) * seg_len + f.u0) * 2);
            if (WHOLE) {
                const uint32_t off = f.ok ? base : kNoWrite;
                __builtin_amdgcn_raw_buffer_store_b128(u32x4{r[0], r[1], r[2], r[3]}, dst, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b128(u32x4{r[4], r[5], r[6], r[7]}, dst, off + (f.ok ? 16 : 0), 0, 0);
            } else {
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const bool keep = f.ok && f.pos + t >= f.lo && f.pos + t < f.hi;
                    __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(r[t >> 1] >> (16 * (t & 1))), dst,
                                                          keep ? base + 2 * t : kNoWrite, 0, 0);
                }
            }
        }
        return;
    }

    const E4m3Quantizer qz = make_quantizer(scale);
    uint64_t nan = 0;
    // r[k]: the 16-token run of dim d0 + k; dword m holds tokens 4m..4m+3
    u32x4 r[DPL];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        float v[4][DPL];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const uint32_t xt = x[4 * m + a];
            const float f0 = lo_f(xt), f1 = hi_f(xt);
            nan |= __builtin_amdgcn_ballot_w64(DPL == 2 ? __builtin_isunordered(f0, f1) : f0 != f0);
            v[a][0] = quotient<FAST>(f0, qz);
            if (DPL == 2)
                v[a][DPL - 1] = quotient<FAST>(f1, qz);
        }
#pragma unroll
        for (int k = 0; k < DPL; ++k)
            r[k][m] = e4m3_pack2<true>(v[2][k], v[3][k], e4m3_pack2<false>(v[0][k], v[1][k], 0u));
    }
    if (nan != 0) {
#pragma unroll
        for (int t = 0; t < 16; ++t)
#pragma unroll
            for (int k = 0; k < DPL; ++k)
                r[k][t >> 2] = e4m3_patch_nan(r[k][t >> 2], t & 3, k ? hi_f(x[t]) : lo_f(x[t]));
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
        const uint32_t base = static_cast<uint32_t>((d0 + k) * seg_len + f.u0);
        if (TILE) {
            *reinterpret_cast<u32x4 *>(lds + (d0 + k) * kFillLdsRow + 16 * f.grp) = r[k];
        } else if (WHOLE) {
            __builtin_amdgcn_raw_buffer_store_b128(r[k], dst, f.ok ? base : kNoWrite, 0, 0);
        } else {
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const bool keep = f.ok && f.pos + t >= f.lo && f.pos + t < f.hi;
                __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(r[k][t >> 2] >> (8 * (t & 3))), dst,
                                                     keep ? base + t : kNoWrite, 0, 0);
            }
        }
    }
}

// A whole e4m3 tile in pages of 64 tokens or more is exactly one V segment:
// the four V waves leave their 16-token runs in LDS, and the work-group then
// stores each head dim's 64-byte row whole, a wave writing 1 KiB of
// consecutive memory per instruction (16-byte runs from four waves would
// each be a separate cache write request).
template <int D>
__device__ __forceinline__ void fill_v_tile_store(const FillGroup &f, const uint8_t *lds)
{
    const auto dst = buffer_at(f.seg);
#pragma unroll
    for (int i = 0; i < D * 4 / (64 * kFillWaves); ++i) {
        const int piece = static_cast<int>(threadIdx.x) + 64 * kFillWaves * i;
        const int dim = piece >> 2, qtr = piece & 3;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + dim * kFillLdsRow + 16 * qtr);
        __builtin_amdgcn_raw_buffer_store_b128(v, dst, static_cast<uint32_t>(dim * 64 + 16 * qtr), 0, 0);
    }
}

template <bool BF16, int D, bool FAST>
__device__ __forceinline__ void fill_group(const FillGroup &f, bool is_v, bool whole, bool tile, float scale,
                                           int lane, uint8_t *lds)
{
    if (is_v) {
        if (tile) {
            fill_v_group<BF16, D, FAST, true, true>(f, scale, lane, lds);
            __syncthreads();
            fill_v_tile_store<D>(f, lds);
        } else if (whole) {
            fill_v_group<BF16, D, FAST, true, false>(f, scale, lane, lds);
        } else {
            fill_v_group<BF16, D, FAST, false, false>(f, scale, lane, lds);
        }
    } else {
        if (whole)
            fill_k_group<BF16, D, FAST, true>(f, scale, lane);
        else
            fill_k_group<BF16, D, FAST, false>(f, scale, lane);
    }
}

template <bool BF16, int D>
__global__ __launch_bounds__(64 * kFillWaves) void kv_fill_kernel(WriteParams p, int tiles_per_req)
{
    constexpr int E = BF16 ? 2 : 1;
    constexpr int LOG2_MAXSEG = BF16 ? 5 : 6;   // 64 bytes per element column
    __shared__ __align__(16) uint8_t lds[D * kFillLdsRow];
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / 64);
    const int lane = threadIdx.x % 64;
    const int half = static_cast<int>(gridDim.x / 2);
    const bool is_v = static_cast<int>(blockIdx.x) >= half;
    const int blk = static_cast<int>(blockIdx.x) - (is_v ? half : 0);
    const int k = blk % tiles_per_req;
    const int bg = blk / tiles_per_req;
    const int g = bg % p.num_kv_heads;
    const int b = bg / p.num_kv_heads;
    if (p.req_status != nullptr && p.req_status[b] != 0)
        return;
    const int T = p.src_tokens;
    const int64_t start = p.token_start[b];
    int64_t count = p.token_count[b];
    if (count > T)
        count = T;
    if (count <= 0)
        return;
    const int64_t cap = static_cast<int64_t>(p.max_pages) << p.log2_page;
    const int64_t pos0 = ((start >> 6) + k) << 6;
    FillGroup f;
    f.lo = pos0 > start ? pos0 : start;
    if (f.lo < 0)
        f.lo = 0;
    f.hi = pos0 + kFillTile;
    if (f.hi > start + count)
        f.hi = start + count;
    if (f.hi > cap)
        f.hi = cap;
    f.pos = pos0 + 16 * wave;
    f.grp = wave;
    if (f.pos + 16 <= f.lo || f.pos >= f.hi)
        return;                                  // then 0 <= pos < cap below
    const bool whole = f.pos >= f.lo && f.pos + 16 <= f.hi;
    int32_t page = p.page_table[static_cast<int64_t>(b) * p.max_pages + (f.pos >> p.log2_page)];
    f.ok = page >= 0 && page < p.num_pages;
    if (!f.ok)
        page = 0;
    f.log2_seg = p.log2_page < LOG2_MAXSEG ? p.log2_page : LOG2_MAXSEG;
    const int slot = static_cast<int>(f.pos & ((int64_t{1} << p.log2_page) - 1));
    f.u0 = slot & ((1 << f.log2_seg) - 1);
    f.seg = (is_v ? p.v_pool : p.k_pool) +
            ((((static_cast<int64_t>(page) * p.num_kv_heads + g) << p.log2_page) + (slot - f.u0)) * D) * E;
    f.row_bytes = p.num_kv_heads * D * 2;
    f.src = reinterpret_cast<const char *>(is_v ? p.v_src : p.k_src) +
            (static_cast<int64_t>(b) * T * p.num_kv_heads + g) * D * 2 + (f.pos - start) * f.row_bytes;
    if (BF16) {
        fill_group<BF16, D, true>(f, is_v, whole, false, 1.0f, lane, lds);
        return;
    }
    // the same on every wave of the work-group: all four groups share the page
    const bool tile = is_v && p.log2_page >= 6 && f.lo == pos0 && f.hi == pos0 + kFillTile && f.ok;
    const float scale = is_v ? p.v_scale[g] : p.k_scale[g];
    if (scale >= 0x1p-64f && scale <= 0x1p64f)
        fill_group<BF16, D, true>(f, is_v, whole, tile, scale, lane, lds);
    else
        fill_group<BF16, D, false>(f, is_v, whole, tile, scale, lane, lds);
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
    // tiles one request's span can touch: ceil(T / 64) + 1 (an unaligned start)
    const int tiles = (p.src_tokens + kFillTile - 1) / kFillTile + 1;
    const int64_t blocks = 2 * static_cast<int64_t>(p.batch) * p.num_kv_heads * tiles;   // K, then V
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((kv_fill_kernel<BF16, D>), dim3(static_cast<unsigned>(blocks)), dim3(64 * kFillWaves),
                       0, stream, p, tiles);
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
