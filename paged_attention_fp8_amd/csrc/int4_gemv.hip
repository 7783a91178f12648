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
// 2 to 16 rows of x (and up to 64 when K is not a multiple of 1024): a
// work-group owns 4 to 8 tiles of 16 output rows (one tile per wave) over
// all of K (int4_gemv_kernel); at 2-16 rows the launch picks the tile count
// that gives every CU the same number of tiles where it can (8-wave
// work-groups, spare waves staging x).  Per group of 128 features the work-group
// stages x[0:16*MT][group] in LDS; each wave expands its 1 KiB block to
// bf16, runs 4 MFMAs per 16-row tile of x and adds s times the group's
// partial sums into its fp32 accumulators.  Up to 32 rows the expansion is
// 136 + q (a shift and one logic op per pair) with the offset taken back
// out by MFMAs against -136; from 33 rows on v_cvt_off_f32_i4 gives q/16
// exactly and the factor 16 goes into the scale.
// 17 to 64 rows with K a multiple of 1024: 32x32 MFMA tiles, a work-group
// of 8 waves per 128 output rows, x loaded straight into LDS
// (int4_gemv_wide_kernel).
// One row of x: a work-group per 16-row tile whose waves split K, with x
// broadcast to the MFMA's 16 rows (int4_gemv_row_kernel).
#include "pafp8_device.hpp"
#include "pafp8_internal.hpp"

namespace pafp8 {
namespace {

constexpr int kGemvWaves = 4;
constexpr int kGemvThreads = 64 * kGemvWaves;
constexpr int kGroup = 128;        // input features per scale
constexpr int kXcds = 8;           // MI355X: work-groups are dealt to 8 XCDs in turn
constexpr int kStreamLoad = 2;     // buffer load policy: non-temporal (weights are read once)

typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

// a wave-uniform address kept in scalar registers (a buffer resource built
// from it otherwise lands in vector registers and every load through it
// becomes a loop over the distinct values)
__device__ __forceinline__ void *uniform_ptr(const void *p)
{
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a)));
    const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32)));
    return reinterpret_cast<void *>(lo | (hi << 32));
}

// v_cvt_off_f32_i4 (q/16 of the low nibble of its operand) reading byte B
// of v: written out because the compiler folds (w >> 4) >> 8i into one
// shift and then cannot use the byte select
template <int B>
__device__ __forceinline__ float cvt_off_byte(uint32_t v)
{
    float f;
    if constexpr (B == 0)
        f = __builtin_amdgcn_cvt_off_f32_i4(v);
    else if constexpr (B == 1)
        asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(f) : "v"(v));
    else if constexpr (B == 2)
        asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(f) : "v"(v));
    else
        asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(f) : "v"(v));
    return f;
}

// 8 int4 weights (one dword, low nibble first) -> 8 bf16 of q/16, exact.
// Nibble 2i is the low half of byte i of w, nibble 2i + 1 that of byte i of
// w >> 4: one shift, eight conversions, four packs.
__device__ __forceinline__ bf16x8 int4x8_to_bf16_div16(uint32_t w)
{
    const uint32_t hi = w >> 4;
    f32x2 f[4];
    f[0][0] = cvt_off_byte<0>(w);
    f[0][1] = cvt_off_byte<0>(hi);
    f[1][0] = cvt_off_byte<1>(w);
    f[1][1] = cvt_off_byte<1>(hi);
    f[2][0] = cvt_off_byte<2>(w);
    f[2][1] = cvt_off_byte<2>(hi);
    f[3][0] = cvt_off_byte<3>(w);
    f[3][1] = cvt_off_byte<3>(hi);
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
// WAVES: waves per work-group; the first tiles_per_wg of them own a tile
// each, and the others (8-wave work-groups owning 5-7 tiles) only help
// stage x, so that a launch can give every CU the same number of tiles.
template <int MT, int PF, bool PLUS136, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void int4_gemv_kernel(
    const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ w,
    const uint16_t *__restrict__ scales, int N, int K, float *__restrict__ y, int tiles_per_wg)
{
    constexpr int THREADS = 64 * WAVES;
    constexpr int XC = MT == 1 ? 4 : (MT == 2 ? 2 : 1);  // groups per staged x chunk
    constexpr int XS = XC * kGroup + 8;                  // LDS row stride (bf16), 16 bytes of padding
    constexpr int XP = MT * XC * kGemvWaves / WAVES;     // 16-byte x pieces per thread per chunk
    static_assert(MT * XC * kGemvWaves % WAVES == 0, "a chunk of x splits evenly over the threads");
    __shared__ __align__(16) uint16_t xs[2][MT * 16 * XS];
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int tid = threadIdx.x;
    const int n_tiles = N / 16;
    const int nt = blockIdx.x * tiles_per_wg + wave;  // this wave's 16-row tile
    const bool owner = wave < tiles_per_wg;           // wave-uniform
    const bool live = owner && nt < n_tiles;
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
            const int idx = tid + it * THREADS;
            const int m = idx / (XC * kGroup / 8), c8 = idx % (XC * kGroup / 8);
            const int mr = m < M ? m : M - 1;
            xr[it] = load16(x + static_cast<int64_t>(mr) * K + static_cast<int64_t>(ch) * XC * kGroup + c8 * 8);
        }
    };
    auto store_x = [&](int buf) {
#pragma unroll
        for (int it = 0; it < XP; ++it) {
            const int idx = tid + it * THREADS;
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

    if (!owner) {
        // a helper wave: the same x staging and barriers as the owners' loop
        load_x(0);
        store_x(0);
        __syncthreads();
        const int last_ch = G / XC - 1;
        for (int ch = 0; ch <= last_ch; ++ch) {
            load_x(ch + 1 <= last_ch ? ch + 1 : last_ch);
            store_x((ch + 1) & 1);
            __syncthreads();
        }
        return;
    }
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

// 33 to 64 rows of x on 32x32 output tiles (v_mfma_f32_32x32x16_bf16).  The
// packed layout is the same as above: for k-step s of a group (features
// 16s .. 16s + 16) the B operand of lane L = 32h + 16t + r is row r of tile t
// of a tile pair at features 16s + 8h .. + 8, i.e. dword s/2 of the 16-byte
// piece at position 16h + r (s even) or 32 + 16h + r (s odd) of that tile's
// block.  Weights expand as q/16 (v_cvt_off_f32_i4) and the factor 16 goes
// into the scale.
// A work-group of 8 waves owns 128 output rows (8 tiles) over all of K:
// wave w takes the 4 tiles of quad w & 1 (two tile pairs) over the quarter
// w >> 1 of K, so each x operand it reads from LDS feeds 64 weight rows, and
// each group of x staged in LDS serves 128.  The quarters' sums meet in LDS
// at the end.
// x goes from memory straight into LDS (buffer loads with the LDS
// destination, 1 KiB per instruction), with no pass through registers.  An
// instruction fills 4 rows of 256 bytes; the 16-byte piece p of row R holds
// x's piece p ^ (R & 15), so the 32 rows one operand read touches spread
// over all banks.
constexpr int kWideWaves = 8;
constexpr int kWideThreads = 64 * kWideWaves;

template <int MT>   // 32-row tiles of x: 1 (up to 32 rows) or 2 (up to 64)
__global__ __launch_bounds__(kWideThreads, 1) void int4_gemv_wide_kernel(
    const uint16_t *__restrict__ x, int M, const uint8_t *w, const uint16_t *scales, int N, int K,
    float *__restrict__ y)
{
    constexpr int PF = 2;                          // groups of weights in flight per wave
    constexpr int XR = 32 * MT;                    // rows of x staged
    constexpr int QTR_BYTES = XR * kGroup * 2;     // one K quarter of a step
    constexpr int BUF_BYTES = 4 * QTR_BYTES;       // one step: all four quarters
    constexpr int CW = BUF_BYTES / 1024 / kWideWaves;   // 1 KiB LDS loads per wave per step
    constexpr int LPS = 3 * 2;                     // weight and scale loads per step (2 tile pairs)
    __shared__ __align__(1024) unsigned char xs[2 * BUF_BYTES];   // [buffer][K quarter][row][256 B]
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int quad = wave & 1, qtr = wave >> 1;
    const int G = K / kGroup, GQ = G / 4;        // groups per K quarter (a multiple of PF)
    const int r = lane & 15, t = (lane >> 4) & 1, h = lane >> 5;
    const int n_tiles = N / 16;
    const int g0 = qtr * GQ;                     // this wave's first group

    // Buffer loads: a wave-uniform base in the resource, per-lane offsets
    // fixed for the whole loop and the group's offset in a scalar register,
    // so stepping through K costs no vector address arithmetic.  Tiles past
    // N read the wave's first tile (clamped into range) and are not stored.
    // Weights and scales are not declared __restrict__: loads from
    // restricted read-only memory may be moved across the inline-asm
    // barriers below, whose waits count them.
    const int tile0 = uniform(min(blockIdx.x * 8 + 4 * quad, n_tiles - 1));
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(w + static_cast<int64_t>(tile0) * G * 1024), 0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t srs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(scales), 0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t xrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(x), 0, 0x7FFFFFFF, 0x00020000);
    int nt[2], wvo[2], svo[2];   // per tile pair: this lane's tile, weight and scale offsets
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
        nt[tp] = blockIdx.x * 8 + 4 * quad + 2 * tp + t;
        const int tl = nt[tp] < n_tiles ? nt[tp] : tile0;
        wvo[tp] = (tl - tile0) * G * 1024 + (16 * h + r) * 16;
        svo[tp] = (tl * 16 + r) * 2;
    }

    f32x16 acc[2][MT];
#pragma unroll
    for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[tp][mt][v] = 0.f;

    // x of step i: rows [0, XR) of groups qq * GQ + i, qq = 0..3.  LDS load j
    // of this wave fills 1 KiB block c = CW * wave + j of the step's buffer:
    // quarter c / (XR / 4), rows 4 (c % (XR / 4)) + lane / 16.  Rows >= M
    // repeat row M - 1: an output row depends on its own row of x alone, and
    // rows >= M are never stored.
    int xvo[CW];
#pragma unroll
    for (int j = 0; j < CW; ++j) {
        const int c = CW * wave + j;
        const int qq = c / (XR / 4), row = 4 * (c % (XR / 4)) + (lane >> 4);
        const int mr = row < M ? row : M - 1;
        xvo[j] = (mr * K + qq * GQ * kGroup + (((lane & 15) ^ (row & 15)) * 8)) * 2;
    }
    // (the offsets are passed as unsigned: given an int, the host pass
    // silently drops the kernel's launch stub)
    auto load_x = [&](int i, int buf) {
#pragma unroll
        for (int j = 0; j < CW; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xrs, (__attribute__((address_space(3))) void *)(xs + buf * BUF_BYTES + (CW * wave + j) * 1024), 16,
                static_cast<unsigned>(xvo[j]), static_cast<unsigned>(i * kGroup * 2), 0, 0);
    };
    // this lane's operand of k-step s (tile mt adds 32 rows = 8 KiB)
    int xrd[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
        xrd[s] = qtr * QTR_BYTES + (lane & 31) * 256 + (((2 * s + h) ^ (lane & 15)) * 16);

    u32x4 wlo[PF][2], whi[PF][2];   // positions 16h + r (even k-steps) and 32 + 16h + r (odd)
    uint32_t sr[PF][2];
    auto load_w = [&](int u, int g) {
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
            wlo[u][tp] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, wvo[tp], g * 1024, kStreamLoad));
            whi[u][tp] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, wvo[tp] + 512, g * 1024, kStreamLoad));
            sr[u][tp] = __builtin_amdgcn_raw_buffer_load_b16(srs, svo[tp], g * N * 2, 0);
        }
    };
    load_x(0, 0);
#pragma unroll
    for (int u = 0; u < PF; ++u)
        load_w(u, g0 + u);
    // x of step 0 in LDS (only the weight loads issued after it may still be
    // in flight), then every wave's.  The scheduling barriers keep the
    // compiler from moving memory operations across the waits.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(LPS * PF) : "memory");
    __builtin_amdgcn_sched_barrier(0);

    for (int i0 = 0; i0 < GQ; i0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int i = i0 + u;
            // buffer (i + 1) & 1 was last read in step i - 1, before the
            // barrier that ended it; after the last step this load is dead
            // but keeps the loop uniform
            load_x(i + 1 < GQ ? i + 1 : GQ - 1, (u + 1) & 1);
            // the step's weight loads must follow these: the wait at the
            // step's end counts on it
            __builtin_amdgcn_sched_barrier(0);
            u32x4 wa[2], wc[2];
            float s16[2];
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
                wa[tp] = wlo[u][tp];
                wc[tp] = whi[u][tp];
                s16[tp] = 16.0f * __uint_as_float(sr[u][tp] << 16);
            }
            load_w(u, g0 + (i + PF < GQ ? i + PF : GQ - 1));
            const unsigned char *xb = xs + (u & 1) * BUF_BYTES;
            f32x16 part[2][MT];
#pragma unroll
            for (int tp = 0; tp < 2; ++tp)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        part[tp][mt][v] = 0.f;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                bf16x8 a[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    a[mt] = *reinterpret_cast<const bf16x8 *>(xb + xrd[s] + mt * 32 * 256);
#pragma unroll
                for (int tp = 0; tp < 2; ++tp) {
                    const bf16x8 b = int4x8_to_bf16_div16((s & 1) ? wc[tp][s >> 1] : wa[tp][s >> 1]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        part[tp][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt], b, part[tp][mt], 0, 0, 0);
                }
            }
#pragma unroll
            for (int tp = 0; tp < 2; ++tp)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[tp][mt] += s16[tp] * part[tp][mt];
            // this wave's x loads of step i + 1 have landed (only the weight
            // loads after them may be outstanding) and its reads of buffer
            // i & 1 are done; the barrier makes that true of all waves
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LPS) : "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // no LDS load may still be in flight where the sums meet
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // the K quarters meet: quarters 1..3 hand their sums to quarter 0
    float *red = reinterpret_cast<float *>(xs);   // [quad][quarter - 1][tp][mt][v][lane]
    constexpr int RW = 2 * MT * 16 * 64;          // floats per wave
    if (qtr > 0) {
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    red[(quad * 3 + qtr - 1) * RW + ((tp * MT + mt) * 16 + v) * 64 + lane] = acc[tp][mt][v];
    }
    __syncthreads();
    if (qtr > 0)
        return;
    // acc[tp][mt][v] = y[32mt + 8(v/4) + 4h + v%4][16 nt[tp] + r]
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
        if (nt[tp] >= n_tiles)
            continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = mt * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                const int o = ((tp * MT + mt) * 16 + v) * 64 + lane;
                if (m < M)
                    y[static_cast<int64_t>(m) * N + nt[tp] * 16 + r] =
                        acc[tp][mt][v] + red[(quad * 3) * RW + o] + red[(quad * 3 + 1) * RW + o] +
                        red[(quad * 3 + 2) * RW + o];
            }
    }
}

// One row of x.  The weights expand as in the PLUS136 path (bf16 pairs
// (136 + q_i, 136 + q_{i+4}), x staged in the same pairing) and x is
// broadcast to all 16 rows of the MFMA's A operand, so every output row of
// the MFMA is y's row and lanes 0..15 read it off.  The offset, 136 times
// the group's sum of x, is one scalar per group, taken out as the group's
// partial sum joins the accumulator.  Against dot-product instructions on
// the VALU this halves the VALU work per weight.
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
    // XCD-aware tiles: work-groups go to the 8 XCDs in turn, so XCD x gets
    // the consecutive tiles [x * per, (x + 1) * per) -- the four tiles whose
    // scales share a 128-byte line are fetched into one L2, not four
    const int n_tiles = N / 16, per = (n_tiles + kXcds - 1) / kXcds;
    const int nt = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    if (nt >= n_tiles)
        return;
    const int G = K / kGroup;
    const int C = G / XC;                                   // chunks of K
    const int c0 = wave * C / kGemvWaves, c1 = (wave + 1) * C / kGemvWaves;
    const int c = lane & 15, kq = lane >> 4;
    const int g_first = c0 * XC, g_last = c1 * XC - 1;      // this wave's groups (none if c0 == c1)

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
    // The expansion's offset, 136 times the sum of x over a group, is the same
    // for every output row (x has one row): one scalar per group of the
    // staged chunk, from the 16 lanes 16u .. 16u + 15 that hold group u.
    float cx[XC];
    auto offsets = [&]() {
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            t += bf16_lo(xr[e]) + bf16_hi(xr[e]);
#pragma unroll
        for (int m = 1; m < 16; m <<= 1)
            t += shfl_xor_f(t, m);
#pragma unroll
        for (int u = 0; u < XC; ++u)
            cx[u] = -136.0f * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 16 * u));
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
        offsets();
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
                }
                tot = __builtin_fmaf(s, part[0] + cx[u], tot);   // part[i]: output row 4kq + i, column c
            }
            // the wave's own LDS: its DS operations run in order, no barrier
            store_x(buf ^ 1);
            offsets();
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
                            int N, int K, float *y, int num_cus, hipStream_t stream)
{
    const int n_tiles = N / 16;
    const dim3 grid((n_tiles + kGemvWaves - 1) / kGemvWaves);
    // 2-16 rows: tiles per work-group (4 to 8) so that the busiest CU holds
    // the fewest tiles, one work-group per CU at a time counted; ties go to
    // more tiles per work-group (x staged fewer times).  28672 rows of
    // weights on 256 CUs: 7 tiles, 256 work-groups, against 448 four-tile
    // work-groups on which three CUs in four hold 8 tiles.
    int tpw = kGemvWaves;
    {
        int64_t best = -1;
        for (int t = 8; t >= kGemvWaves; --t) {
            const int64_t wgs = (n_tiles + t - 1) / t;
            const int64_t busiest = (wgs + num_cus - 1) / num_cus * t;
            if (best < 0 || busiest < best) {
                best = busiest;
                tpw = t;
            }
        }
    }
    const int mt = (M + 15) / 16;
    const bool pf8 = (K / kGroup) % 8 == 0;   // K % 512 == 0 gives a multiple of 4
    if (M == 1) {
        const int per = (n_tiles + kXcds - 1) / kXcds;
        hipLaunchKernelGGL(int4_gemv_row_kernel, dim3(per * kXcds), dim3(kGemvThreads), 0, stream, x, w,
                           scales, N, K, y);
        return hipGetLastError();
    }
#define PAFP8_GEMV(MT_)                                                                            \
    if (pf8)                                                                                       \
        hipLaunchKernelGGL((int4_gemv_kernel<MT_, 8, (MT_ <= 2), kGemvWaves>), grid, dim3(kGemvThreads), 0, \
                           stream, x, M, w, scales, N, K, y, kGemvWaves);                         \
    else                                                                                           \
        hipLaunchKernelGGL((int4_gemv_kernel<MT_, 4, (MT_ <= 2), kGemvWaves>), grid, dim3(kGemvThreads), 0, \
                           stream, x, M, w, scales, N, K, y, kGemvWaves);
    // 17-64 rows on 32x32 tiles (K a multiple of 1024: whole prefetch rings
    // in each quarter of K; and 32-bit buffer offsets into x and the scales)
    const bool wide = (K / kGroup / 4) % 2 == 0 && static_cast<int64_t>(K) * 64 * 2 < INT32_MAX &&
                      static_cast<int64_t>(K / kGroup + 1) * N * 2 < INT32_MAX;
    if (mt == 1 && tpw > kGemvWaves) {
        const dim3 grid8((n_tiles + tpw - 1) / tpw);
        if (pf8)
            hipLaunchKernelGGL((int4_gemv_kernel<1, 8, true, 8>), grid8, dim3(8 * 64), 0, stream, x, M, w,
                               scales, N, K, y, tpw);
        else
            hipLaunchKernelGGL((int4_gemv_kernel<1, 4, true, 8>), grid8, dim3(8 * 64), 0, stream, x, M, w,
                               scales, N, K, y, tpw);
    } else if (mt == 1) {
        PAFP8_GEMV(1)
    } else if (mt == 2 && wide) {
        hipLaunchKernelGGL((int4_gemv_wide_kernel<1>), dim3((n_tiles + 7) / 8), dim3(kWideThreads), 0, stream, x,
                           M, w, scales, N, K, y);
    } else if (mt == 2) {
        PAFP8_GEMV(2)
    } else if (wide) {
        hipLaunchKernelGGL((int4_gemv_wide_kernel<2>), dim3((n_tiles + 7) / 8), dim3(kWideThreads), 0, stream, x,
                           M, w, scales, N, K, y);
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
