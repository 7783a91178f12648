// int4_gemv.hip -- decode-time weight streaming with INT4 weights,
// dequantized on read.
//
// Cloudflare, "Smaller, faster, safer: running Kimi and GLM at scale",
// section "模型权重压缩" (model weight compression: GLM weights FP8 -> INT4): decode
// streams the weights from GPU memory for every generated token, so 4-bit
// weights move fewer bytes and decode runs faster; the weights are expanded
// before the multiplication.  The pages give no grouping or zero point; the
// reading here is symmetric signed 4-bit integers q in [-8, 7] with one bf16
// scale per 128 consecutive input features of an output row:
//     y[m][n] = sum_k x[m][k] * q[n][k] * s[k / 128][n].
//
// Packed weight layout (include/pafp8.h): 1 KiB blocks of 16 output rows x
// 128 input features, ordered [N / 16][K / 128].  Lane L = 16*kq + c of a
// wave loads the 16 bytes at L*16 of a block; their dword j holds the 8
// weights of row c at features 32j + 8kq .. +8 (feature order = nibble
// order, low nibble first), which is exactly lane L's B operand of the j-th
// v_mfma_f32_16x16x32_bf16 over the block.
//
// Two rows of x or more: a work-group of 4 waves owns 64 output rows (one
// 16-row tile per wave) over all of K.  Per group of 128 features the
// work-group stages x[0:16*MT][group] in LDS; each wave expands its 1 KiB
// block to bf16, runs 4 MFMAs per 16-row tile of x and adds s times the
// group's partial sums into its fp32 accumulators.  Up to 32 rows the
// expansion is 136 + q (a shift and one logic op per pair) with the offset
// taken back out by MFMAs against -136; from 33 rows on v_cvt_off_f32_i4
// gives q/16 exactly and the factor 16 goes into the scale.
// One row of x: a work-group per 16-row tile whose waves split K, with x
// broadcast to the MFMA's 16 rows (int4_gemv_row_kernel).
#include "pafp8_device.hpp"
#include "pafp8_internal.hpp"

namespace pafp8 {
namespace {

constexpr int kGemvWaves = 4;
constexpr int kGemvThreads = 64 * kGemvWaves;
constexpr int kGroup = 128;        // input features per scale

// 8 int4 weights (one dword, low nibble first) -> 8 bf16 of q/16, exact
__device__ __forceinline__ bf16x8 int4x8_to_bf16_div16(uint32_t w)
{
    f32x2 f[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i][0] = __builtin_amdgcn_cvt_off_f32_i4(w >> (8 * i));
        f[i][1] = __builtin_amdgcn_cvt_off_f32_i4(w >> (8 * i + 4));
    }
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2 p = __builtin_convertvector(f[i], bf16x2);
        r[2 * i] = p[0];
        r[2 * i + 1] = p[1];
    }
    return r;
}

// 8 int4 weights (one dword) -> the bf16 pairs (136 + q_i, 136 + q_{i+4}),
// i = 0..3: ((w >> 4i) & 0x000F000F) ^ 0x43084308 flips the nibble's top bit
// (q + 8 < 16) and puts it under the exponent of 128, a shift and one logic
// operation per pair
__device__ __forceinline__ bf16x8 int4x8_to_bf16_plus136(uint32_t w)
{
    u32x4 t;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        t[i] = ((w >> (4 * i)) & 0x000F000Fu) ^ 0x43084308u;
    return __builtin_bit_cast(bf16x8, t);
}

// MT: 16-row tiles of x; PF: weight blocks in flight per wave, a divisor of
// K / 128 (so the unrolled group loop needs no early exit, which would let
// the compiler sink the x loads to their use).  PLUS136: weights expanded as
// 136 + q (fewer VALU operations, features of each 8-block paired (i, i+4) in
// both operands) and the 136 taken back out by MFMAs of the same x against a
// constant -136, which the matrix cores absorb while they idle at few rows.
template <int MT, int PF, bool PLUS136>
__global__ __launch_bounds__(kGemvThreads) void int4_gemv_kernel(
    const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ w,
    const uint16_t *__restrict__ scales, int N, int K, float *__restrict__ y)
{
    constexpr int XC = MT == 1 ? 4 : (MT == 2 ? 2 : 1);  // groups per staged x chunk
    constexpr int XS = XC * kGroup + 8;                  // LDS row stride (bf16), 16 bytes of padding
    constexpr int XP = MT * XC;                          // 16-byte x pieces per thread per chunk
    __shared__ __align__(16) uint16_t xs[2][MT * 16 * XS];
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int tid = threadIdx.x;
    const int n_tiles = N / 16;
    const int nt = blockIdx.x * kGemvWaves + wave;  // this wave's 16-row tile
    const bool live = nt < n_tiles;
    const int G = K / kGroup;
    const int c = lane & 15, kq = lane >> 4;

    // x chunk ch: rows [0, 16*MT) x features [ch*XC*128, (ch+1)*XC*128); rows
    // >= M are zero.  Loads in the main loop are unconditional (rows and
    // blocks clamped into range, unwanted values dropped by a select): a
    // conditional load would make the compiler wait for it where the
    // branches join.
    u32x4 xr[XP];
    auto load_x = [&](int ch) {
#pragma unroll
        for (int it = 0; it < XP; ++it) {
            const int idx = tid + it * kGemvThreads;
            const int m = idx / (XC * kGroup / 8), c8 = idx % (XC * kGroup / 8);
            const int mr = m < M ? m : M - 1;
            xr[it] = load16(x + static_cast<int64_t>(mr) * K + static_cast<int64_t>(ch) * XC * kGroup + c8 * 8);
        }
    };
    auto store_x = [&](int buf) {
#pragma unroll
        for (int it = 0; it < XP; ++it) {
            const int idx = tid + it * kGemvThreads;
            const int m = idx / (XC * kGroup / 8), c8 = idx % (XC * kGroup / 8);
            u32x4 v = m < M ? xr[it] : u32x4{0u, 0u, 0u, 0u};
            if (PLUS136) {
                const u32x4 a = v;
                v[0] = __builtin_amdgcn_perm(a[2], a[0], 0x05040100u);   // features 0, 4
                v[1] = __builtin_amdgcn_perm(a[2], a[0], 0x07060302u);   // 1, 5
                v[2] = __builtin_amdgcn_perm(a[3], a[1], 0x05040100u);   // 2, 6
                v[3] = __builtin_amdgcn_perm(a[3], a[1], 0x07060302u);   // 3, 7
            }
            *reinterpret_cast<u32x4 *>(&xs[buf][m * XS + c8 * 8]) = v;
        }
    };

    const uint8_t *wb = w + (static_cast<int64_t>(live ? nt : 0) * G) * 1024 + lane * 16;
    const uint16_t *sp = scales + (live ? nt : 0) * 16 + c;
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // scales kept one per 32-bit register: packing two 16-bit values per
    // register would make the compiler wait for each scale load at once
    u32x4 wr[PF];
    uint32_t sr[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        const int gl = u < G ? u : G - 1;
        wr[u] = load16_stream(wb + static_cast<int64_t>(gl) * 1024);
        sr[u] = static_cast<uint32_t>(sp[static_cast<int64_t>(gl) * N]);
    }
    load_x(0);
    store_x(0);
    __syncthreads();

    // PF divides G and XC divides PF, so chunk boundaries fall on fixed u
    for (int g0 = 0; g0 < G; g0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int g = g0 + u;
            const int ch = g / XC;
            const int last_ch = G / XC - 1;
            if (u % XC == 0) {
                load_x(ch + 1 <= last_ch ? ch + 1 : last_ch);
                // keep these loads ahead of the chunk's weight loads: the
                // LDS store at the chunk's end then waits for them alone
                __builtin_amdgcn_sched_barrier(0);
            }
            bf16x8 bop[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bop[j] = PLUS136 ? int4x8_to_bf16_plus136(wr[u][j]) : int4x8_to_bf16_div16(wr[u][j]);
            const float s16 = (PLUS136 ? 1.0f : 16.0f) * __uint_as_float(sr[u] << 16);
            {
                const int gl = g + PF < G ? g + PF : G - 1;
                wr[u] = load16_stream(wb + static_cast<int64_t>(gl) * 1024);
                sr[u] = static_cast<uint32_t>(sp[static_cast<int64_t>(gl) * N]);
            }
            const uint16_t *xa = &xs[ch & 1][c * XS + (u % XC) * kGroup + 8 * kq];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(xa + mt * 16 * XS + 32 * j);
                    part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bop[j], part, 0, 0, 0);
                    if (PLUS136) {
                        const bf16x8 neg136 = __builtin_bit_cast(bf16x8, u32x4{0xC308C308u, 0xC308C308u,
                                                                               0xC308C308u, 0xC308C308u});
                        part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, neg136, part, 0, 0, 0);
                    }
                }
                acc[mt] += s16 * part;
            }
            if (u % XC == XC - 1) {
                // every wave is done with buffer (ch + 1) & 1 since the last
                // barrier; after the last chunk this store is dead but keeps
                // the x loads unconditional (and so issued early)
                store_x((ch + 1) & 1);
                __syncthreads();
            }
        }
    }
    if (!live)
        return;
    // acc[mt][i] = y[16*mt + 4*kq + i][16*nt + c]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = mt * 16 + 4 * kq + i;
            if (m < M)
                y[static_cast<int64_t>(m) * N + nt * 16 + c] = acc[mt][i];
        }
}

// One row of x.  The weights expand as in the PLUS136 path (bf16 pairs
// (136 + q_i, 136 + q_{i+4}), x staged in the same pairing) and x is
// broadcast to all 16 rows of the MFMA's A operand, so every output row of
// the MFMA is y's row and lanes 0..15 read it off; a second MFMA of the same
// x against a constant -136 takes the offset back out.  Against dot-product
// instructions on the VALU this halves the VALU work per weight, and the
// matrix cores, otherwise idle, absorb the rest.
//
// A work-group owns one 16-row tile; its four waves take consecutive quarters
// of K (in chunks of 4 groups), each with its own prefetch ring and its own
// x staging, so no wave waits for another until the final sum.
__global__ __launch_bounds__(kGemvThreads) void int4_gemv_row_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ w, const uint16_t *__restrict__ scales,
    int N, int K, float *__restrict__ y)
{
    constexpr int PF = 4;   // weight blocks in flight per wave (one chunk)
    constexpr int XC = 4;   // groups per staged x chunk: one 16-byte piece per lane
    __shared__ __align__(16) uint32_t xs[kGemvWaves][2][XC * kGroup / 2];  // bf16 pairs (x_i, x_{i+4})
    __shared__ float red[kGemvWaves][16];
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int nt = blockIdx.x;
    const int G = K / kGroup;
    const int C = G / XC;                                   // chunks of K
    const int c0 = wave * C / kGemvWaves, c1 = (wave + 1) * C / kGemvWaves;
    const int c = lane & 15, kq = lane >> 4;
    const int g_first = c0 * XC, g_last = c1 * XC - 1;      // this wave's groups (none if c0 == c1)
    const bf16x8 neg136 = __builtin_bit_cast(bf16x8, u32x4{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u});

    u32x4 xr;
    auto load_x = [&](int ch) {
        xr = load16(x + static_cast<int64_t>(ch) * XC * kGroup + lane * 8);
    };
    auto store_x = [&](int buf) {
        u32x4 v;
        v[0] = __builtin_amdgcn_perm(xr[2], xr[0], 0x05040100u);   // features 0, 4
        v[1] = __builtin_amdgcn_perm(xr[2], xr[0], 0x07060302u);   // 1, 5
        v[2] = __builtin_amdgcn_perm(xr[3], xr[1], 0x05040100u);   // 2, 6
        v[3] = __builtin_amdgcn_perm(xr[3], xr[1], 0x07060302u);   // 3, 7
        *reinterpret_cast<u32x4 *>(&xs[wave][buf][lane * 4]) = v;
    };

    float tot = 0.f;
    if (c0 < c1) {
        const uint8_t *wb = w + static_cast<int64_t>(nt) * G * 1024 + lane * 16;
        const uint16_t *sp = scales + nt * 16 + c;
        u32x4 wr[PF];
        uint32_t sr[PF];
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            wr[u] = load16_stream(wb + static_cast<int64_t>(g_first + u) * 1024);
            sr[u] = static_cast<uint32_t>(sp[static_cast<int64_t>(g_first + u) * N]);
        }
        load_x(c0);
        store_x(0);
        for (int ch = c0; ch < c1; ++ch) {
            const int buf = (ch - c0) & 1;
            load_x(ch + 1 < c1 ? ch + 1 : ch);   // unconditional: clamped into this wave's range
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                const int g = ch * XC + u;
                const u32x4 wq = wr[u];
                const float s = __uint_as_float(sr[u] << 16);
                {
                    const int gl = g + PF <= g_last ? g + PF : g_last;
                    wr[u] = load16_stream(wb + static_cast<int64_t>(gl) * 1024);
                    sr[u] = static_cast<uint32_t>(sp[static_cast<int64_t>(gl) * N]);
                }
                // lane (c, kq) feeds features 32j + 8kq .. + 8 of the group
                f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x8 a = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const u32x4 *>(&xs[wave][buf][(u * 16 + 4 * j + kq) * 4]));
                    part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, int4x8_to_bf16_plus136(wq[j]), part, 0, 0, 0);
                    part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, neg136, part, 0, 0, 0);
                }
                tot = __builtin_fmaf(s, part[0], tot);   // part[i]: output row 4kq + i, column c
            }
            // the wave's own LDS: its DS operations run in order, no barrier
            store_x(buf ^ 1);
        }
    }
    if (kq == 0)
        red[wave][c] = tot;
    __syncthreads();
    if (wave == 0 && lane < 16)
        y[nt * 16 + c] = red[0][c] + red[1][c] + red[2][c] + red[3][c];
}

// row-major int4 [N][K/2] -> packed blocks: a permutation of 4-byte words
__global__ __launch_bounds__(256) void int4_pack_kernel(const uint32_t *__restrict__ src,
                                                        uint32_t *__restrict__ dst, int N, int K)
{
    const int64_t words = static_cast<int64_t>(N) * K / 8;
    const int G = K / kGroup;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < words;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        // destination word i: block (nt, g), lane L = 16*kq + c, dword j
        const int j = static_cast<int>(i & 3);
        const int L = static_cast<int>((i >> 2) & 63);
        const int64_t blk = i >> 8;
        const int g = static_cast<int>(blk % G);
        const int64_t nt = blk / G;
        const int c = L & 15, kq = L >> 4;
        const int64_t n = nt * 16 + c;
        const int64_t k = static_cast<int64_t>(g) * kGroup + 32 * j + 8 * kq;
        dst[i] = src[(n * K + k) / 8];
    }
}

}  // namespace

hipError_t launch_int4_gemv(const uint16_t *x, int M, const uint8_t *w, const uint16_t *scales,
                            int N, int K, float *y, hipStream_t stream)
{
    const int n_tiles = N / 16;
    const dim3 grid((n_tiles + kGemvWaves - 1) / kGemvWaves);
    const int mt = (M + 15) / 16;
    const bool pf8 = (K / kGroup) % 8 == 0;   // K % 512 == 0 gives a multiple of 4
    if (M == 1) {
        hipLaunchKernelGGL(int4_gemv_row_kernel, dim3(n_tiles), dim3(kGemvThreads), 0, stream, x, w,
                           scales, N, K, y);
        return hipGetLastError();
    }
#define PAFP8_GEMV(MT_)                                                                            \
    if (pf8)                                                                                       \
        hipLaunchKernelGGL((int4_gemv_kernel<MT_, 8, (MT_ <= 2)>), grid, dim3(kGemvThreads), 0, stream, \
                           x, M, w, scales, N, K, y);                                             \
    else                                                                                           \
        hipLaunchKernelGGL((int4_gemv_kernel<MT_, 4, (MT_ <= 2)>), grid, dim3(kGemvThreads), 0, stream, \
                           x, M, w, scales, N, K, y);
    if (mt == 1) {
        PAFP8_GEMV(1)
    } else if (mt == 2) {
        PAFP8_GEMV(2)
    } else if (mt == 3) {
        PAFP8_GEMV(3)
    } else {
        PAFP8_GEMV(4)
    }
#undef PAFP8_GEMV
    return hipGetLastError();
}

hipError_t launch_int4_pack(const uint8_t *src, uint8_t *dst, int N, int K, hipStream_t stream)
{
    const int64_t words = static_cast<int64_t>(N) * K / 8;
    int64_t blocks = (words + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(int4_pack_kernel, dim3(static_cast<unsigned>(blocks < 1 ? 1 : blocks)), dim3(256), 0,
                       stream, reinterpret_cast<const uint32_t *>(src), reinterpret_cast<uint32_t *>(dst), N, K);
    return hipGetLastError();
}

}  // namespace pafp8
