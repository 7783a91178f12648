// splitk_combine.hip -- the log-sum-exp merge of split-K (flash-decoding)
// partials: per (request, query head), over the splits s with lse_s > -inf,
//     LSE = log sum_s exp(lse_s),   out = sum_s exp(lse_s - LSE) * o_s,
// where o_s is the split's normalised output.  Aborted requests (non-zero
// status) give out = 0, lse = -inf; a NaN partial gives NaN.  The pages do
// not describe splitting; it is how one decode step spreads one long
// request over the GPU, and the merge is exact up to fp32 rounding.
#include "pafp8_device.hpp"
#include "pafp8_internal.hpp"

namespace pafp8 {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kNegInf = -__builtin_huge_valf();

// split-K combine, any head dim (a multiple of 4 up to 1024): one work-group
// per (request, query head).  Threads split the head dims four at a time and
// the splits among themselves; partial sums meet in LDS.
// ===========================================================================
__device__ __forceinline__ float block_reduce(float v, float *red, bool is_max)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = is_max ? wave_max(v) : wave_sum(v);
    __syncthreads();  // red may still be read by a previous reduction
    if (lane == 0)
        red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i)
        r = is_max ? __builtin_fmaxf(r, red[i]) : r + red[i];
    return r;
}

__global__ __launch_bounds__(kThreads) void splitk_combine_kernel(
    const float *__restrict__ part_o, const float *__restrict__ part_lse, int Hq, int S, int D,
    const int32_t *__restrict__ req_status, float *__restrict__ out, float *__restrict__ lse_out)
{
    __shared__ float red[kWaves];
    __shared__ f32x4 acc_sm[kThreads];
    const int bh = blockIdx.x;
    const int b = bh / Hq;
    const float *pl = part_lse + static_cast<int64_t>(bh) * S;
    const float *po = part_o + static_cast<int64_t>(bh) * S * D;
    float *o = out + static_cast<int64_t>(bh) * D;
    const int nd4 = D / 4;                 // float4 columns
    const int ngrp = kThreads / nd4;       // split groups (>= 1 since D <= 1024)
    const int col = threadIdx.x % nd4, grp = threadIdx.x / nd4;

    const bool aborted = req_status != nullptr && req_status[b] != 0;
    float M = kNegInf;
    int has_nan = 0;
    for (int k = threadIdx.x; k < S; k += kThreads) {
        const float v = pl[k];
        has_nan |= v != v;
        M = __builtin_fmaxf(M, v);
    }
    M = block_reduce(M, red, true);
    has_nan = __syncthreads_or(has_nan);
    if (aborted || has_nan || M == kNegInf) {
        const float fill = (has_nan && !aborted) ? __builtin_nanf("") : 0.f;
        for (int d = threadIdx.x; d < D; d += kThreads)
            o[d] = fill;
        if (threadIdx.x == 0 && lse_out != nullptr)
            lse_out[bh] = (has_nan && !aborted) ? fill : kNegInf;
        return;
    }
    float sum = 0.f;
    for (int k = threadIdx.x; k < S; k += kThreads)
        sum += __expf(pl[k] - M);
    sum = block_reduce(sum, red, false);
    const float LSE = M + __logf(sum);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (grp < ngrp) {
        for (int k = grp; k < S; k += ngrp) {
            const float lk = pl[k];
            if (lk == kNegInf)
                continue;  // empty split: contributes nothing
            acc += __expf(lk - LSE) * *reinterpret_cast<const f32x4 *>(po + static_cast<int64_t>(k) * D + col * 4);
        }
    }
    acc_sm[threadIdx.x] = acc;
    __syncthreads();
    if (static_cast<int>(threadIdx.x) < nd4) {
        f32x4 t = acc_sm[threadIdx.x];
        for (int gi = 1; gi < ngrp; ++gi)
            t += acc_sm[gi * nd4 + threadIdx.x];
        *reinterpret_cast<f32x4 *>(o + threadIdx.x * 4) = t;
    }
    if (threadIdx.x == 0 && lse_out != nullptr)
        lse_out[bh] = LSE;
}

// one output row of D floats (and its lse unless lse is nullptr) set by a wave
template <int D>
__device__ __forceinline__ void fill_row(float *o, float *lse, float v, float lse_v)
{
    constexpr int NC = D / 4;
    const int lane = threadIdx.x & 63;
    if (lane < NC)
        *reinterpret_cast<f32x4 *>(o + lane * 4) = f32x4{v, v, v, v};
    if (lane == 0 && lse != nullptr)
        *lse = lse_v;
}

// Wave-per-head combine for the attention's own head dims: one wave merges
// the S partial rows po[S][D] (LSEs pl[S]) of one (request, query head) into
// o (and *lse unless lse is nullptr); lane (g, c) handles float4 column c of
// the rows k = g (mod 64 / (D/4)).  The first PF partial rows of every lane are
// loaded together with the LSEs, so the whole reduction costs one memory
// round trip when S * D <= 64 * 4 * PF (PF = 8 covers 16 splits of 128 dims,
// PF = 32 covers 64).
template <int D, int PF>
__device__ __forceinline__ void combine_rows(const float *__restrict__ pl, const float *__restrict__ po,
                                             int S, bool aborted, float *__restrict__ o,
                                             float *__restrict__ lse)
{
    constexpr int NC = D / 4;    // float4 columns of a row
    constexpr int NG = 64 / NC;  // row groups in a wave
    const int lane = threadIdx.x & 63;
    const int col = lane % NC, grp = lane / NC;
    po += col * 4;
    f32x4 pre[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        const int k = grp + i * NG;
        pre[i] = k < S ? *reinterpret_cast<const f32x4 *>(po + static_cast<int64_t>(k) * D)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float l0 = lane < S ? pl[lane] : kNegInf;
    float M = l0;
    bool nan = l0 != l0;
    for (int k = lane + 64; k < S; k += 64) {
        const float v = pl[k];
        nan |= v != v;
        M = __builtin_fmaxf(M, v);
    }
    M = wave_max(M);
    const bool has_nan = __builtin_amdgcn_ballot_w64(nan) != 0;
    if (aborted || has_nan || M == kNegInf) {
        const float fill = (has_nan && !aborted) ? __builtin_nanf("") : 0.f;
        fill_row<D>(o, lse, fill, (has_nan && !aborted) ? fill : kNegInf);
        return;
    }
    float sum = lane < S ? __expf(l0 - M) : 0.f;
    for (int k = lane + 64; k < S; k += 64)
        sum += __expf(pl[k] - M);
    sum = wave_sum(sum);
    const float LSE = M + __logf(sum);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        const int k = grp + i * NG;
        const float from_lane = __shfl(l0, k & 63, 64);  // every lane takes part
        if (k < S) {
            const float lk = S <= 64 ? from_lane : pl[k];
            if (lk != kNegInf)  // empty split: contributes nothing
                acc += __expf(lk - LSE) * pre[i];
        }
    }
    // the remaining rows, PF at a time: all loads of a batch go out together
    for (int k0 = grp + PF * NG; k0 < S; k0 += PF * NG) {
        f32x4 rows[PF];
        float lks[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const int k = k0 + i * NG < S ? k0 + i * NG : S - 1;   // clamped: no conditional loads
            rows[i] = *reinterpret_cast<const f32x4 *>(po + static_cast<int64_t>(k) * D);
            lks[i] = pl[k];
        }
#pragma unroll
        for (int i = 0; i < PF; ++i)
            if (k0 + i * NG < S && lks[i] != kNegInf)
                acc += __expf(lks[i] - LSE) * rows[i];
    }
#pragma unroll
    for (int m = NC; m < 64; m <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc[e] += shfl_xor_f(acc[e], m);
    }
    if (grp == 0)
        *reinterpret_cast<f32x4 *>(o + col * 4) = acc;
    if (lane == 0 && lse != nullptr)
        *lse = LSE;
}

// Many splits (16 < S <= 256): a work-group per (request, query head), its
// wave w taking the consecutive splits [w C, (w + 1) C), C = ceil(S / 4), so
// that each lane holds a quarter of the rows it would alone.  The waves'
// maxima, then their sums of exp(lse_s - max), meet in LDS; each wave then
// weighs its own rows and wave 0 adds the four partial rows in wave order.
template <int D>
__global__ __launch_bounds__(kThreads) void splitk_combine_wg_kernel(
    const float *__restrict__ part_o, const float *__restrict__ part_lse, int Hq, int S,
    const int32_t *__restrict__ req_status, float *__restrict__ out, float *__restrict__ lse_out)
{
    constexpr int NC = D / 4;    // float4 columns of a row
    constexpr int NG = 64 / NC;  // row groups in a wave
    constexpr int PF = 8;        // rows per lane loaded up front
    __shared__ float sm_m[kWaves], sm_sum[kWaves];
    __shared__ int sm_nan[kWaves];
    __shared__ f32x4 sm_acc[kWaves][NC];
    const int bh = blockIdx.x;
    const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int col = lane % NC, grp = lane / NC;
    const int C = (S + kWaves - 1) / kWaves;
    const int k0 = wave * C;
    const int n = S - k0 < C ? (S - k0 > 0 ? S - k0 : 0) : C;   // this wave's splits (<= 64)
    const float *pl = part_lse + static_cast<int64_t>(bh) * S + k0;
    const float *po = part_o + (static_cast<int64_t>(bh) * S + k0) * D + col * 4;
    f32x4 pre[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        const int k = grp + i * NG;
        pre[i] = k < n ? *reinterpret_cast<const f32x4 *>(po + static_cast<int64_t>(k) * D)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float l0 = lane < n ? pl[lane] : kNegInf;
    const float Mw = wave_max(l0);
    const bool nan_w = __builtin_amdgcn_ballot_w64(l0 != l0) != 0;
    if (lane == 0) {
        sm_m[wave] = Mw;
        sm_nan[wave] = nan_w;
    }
    __syncthreads();
    float M = sm_m[0];
    bool has_nan = sm_nan[0] != 0;
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        M = __builtin_fmaxf(M, sm_m[w]);
        has_nan |= sm_nan[w] != 0;
    }
    const bool aborted = req_status != nullptr && req_status[bh / Hq] != 0;
    float *o = out + static_cast<int64_t>(bh) * D;
    float *lse = lse_out != nullptr ? lse_out + bh : nullptr;
    if (aborted || has_nan || M == kNegInf) {
        if (wave == 0) {
            const float fill = (has_nan && !aborted) ? __builtin_nanf("") : 0.f;
            fill_row<D>(o, lse, fill, (has_nan && !aborted) ? fill : kNegInf);
        }
        return;
    }
    const float sw = wave_sum(lane < n ? __expf(l0 - M) : 0.f);
    if (lane == 0)
        sm_sum[wave] = sw;
    __syncthreads();
    float sum = sm_sum[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
        sum += sm_sum[w];
    const float LSE = M + __logf(sum);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        const int k = grp + i * NG;
        const float lk = __shfl(l0, k & 63, 64);  // every lane takes part
        if (k < n && lk != kNegInf)               // empty split: contributes nothing
            acc += __expf(lk - LSE) * pre[i];
    }
    // rows past the first PF per lane, PF at a time (all loads of a batch
    // go out together; the LSEs come from memory, since lanes leave this
    // loop at different trips and a shuffle may not read an idle lane)
    for (int kb = grp + PF * NG; kb < n; kb += PF * NG) {
        f32x4 rows[PF];
        float lks[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const int k = kb + i * NG < n ? kb + i * NG : n - 1;   // clamped: no conditional loads
            rows[i] = *reinterpret_cast<const f32x4 *>(po + static_cast<int64_t>(k) * D);
            lks[i] = pl[k];
        }
#pragma unroll
        for (int i = 0; i < PF; ++i)
            if (kb + i * NG < n && lks[i] != kNegInf)
                acc += __expf(lks[i] - LSE) * rows[i];
    }
#pragma unroll
    for (int m = NC; m < 64; m <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc[e] += shfl_xor_f(acc[e], m);
    }
    if (grp == 0)
        sm_acc[wave][col] = acc;
    __syncthreads();
    if (wave == 0 && lane < NC) {
        f32x4 t = sm_acc[0][lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            t += sm_acc[w][lane];
        *reinterpret_cast<f32x4 *>(o + lane * 4) = t;
    }
    if (threadIdx.x == 0 && lse != nullptr)
        *lse = LSE;
}

// split-K partials: rows [B][Hq][S]
template <int D, int PF>
__global__ __launch_bounds__(kThreads) void splitk_combine_wave_kernel(
    const float *__restrict__ part_o, const float *__restrict__ part_lse, int BH, int Hq, int S,
    const int32_t *__restrict__ req_status, float *__restrict__ out, float *__restrict__ lse_out)
{
    const int bh = blockIdx.x * kWaves + uniform(threadIdx.x >> 6);
    if (bh >= BH)
        return;
    const bool aborted = req_status != nullptr && req_status[bh / Hq] != 0;
    const int64_t row0 = static_cast<int64_t>(bh) * S;
    combine_rows<D, PF>(part_lse + row0, part_o + row0 * D, S, aborted,
                        out + static_cast<int64_t>(bh) * D, lse_out != nullptr ? lse_out + bh : nullptr);
}

// Balanced-partition partials (decode_attn.hip): request b's pieces are rows
// b + w_first .. b + w_last of its query head's [R] rows, w_first and w_last
// following from the request's first page ps in the sequence and the pages per
// work-group C (prefix[b], prefix[B]).  A request inside one range was
// written whole by the attention kernel; requests with no pages (aborted,
// empty, invalid length) get their fixed outputs here.
template <int D>
__global__ __launch_bounds__(kThreads) void bal_combine_wave_kernel(
    const float *__restrict__ part_o, const float *__restrict__ part_lse,
    const int64_t *__restrict__ prefix, int B, int Hq, int R, const int32_t *__restrict__ req_status,
    const int32_t *__restrict__ context_lens, int max_pages, int log2_page, float *__restrict__ out,
    float *__restrict__ lse_out)
{
    const int bh = blockIdx.x * kWaves + uniform(threadIdx.x >> 6);
    if (bh >= B * Hq)
        return;
    const int b = bh / Hq, h = bh % Hq;
    float *o = out + static_cast<int64_t>(bh) * D;
    float *lse = lse_out != nullptr ? lse_out + bh : nullptr;
    // all four loads go out together (prefix holds an entry for every request)
    const bool aborted = req_status != nullptr && req_status[b] != 0;
    const int64_t L = context_lens[b];
    const int64_t ps = prefix[b], C = prefix[B];
    const bool invalid = L < 0 || L > (static_cast<int64_t>(max_pages) << log2_page);
    if (aborted || invalid || L == 0) {
        const float v = aborted || !invalid ? 0.f : __builtin_nanf("");
        fill_row<D>(o, lse, v, aborted || !invalid ? kNegInf : v);
        return;
    }
    const int64_t n = (L + (int64_t{1} << log2_page) - 1) >> log2_page;
    const int64_t w0 = ps / C, w1 = (ps + n - 1) / C;
    if (w0 == w1)
        return;
    const int64_t row0 = static_cast<int64_t>(h) * R + b + w0;
    combine_rows<D, 8>(part_lse + row0, part_o + row0 * D, static_cast<int>(w1 - w0 + 1), false, o, lse);
}

template <int D>
void launch_combine_wave(const float *part_o, const float *part_lse, int BH, int Hq, int S,
                         const int32_t *req_status, float *out, float *lse, hipStream_t stream)
{
    // up to 16 splits: a wave per (request, head), 8 rows per lane up
    // front; 17 to 256: a work-group per (request, head), the splits in four
    // parts; more: a wave per (request, head), 32 rows per lane at a time
    const dim3 grid(static_cast<unsigned>((BH + kWaves - 1) / kWaves)), block(kThreads);
    if (S <= 16)
        hipLaunchKernelGGL((splitk_combine_wave_kernel<D, 8>), grid, block, 0, stream, part_o, part_lse,
                           BH, Hq, S, req_status, out, lse);
    else if (S <= 4 * 64)
        hipLaunchKernelGGL((splitk_combine_wg_kernel<D>), dim3(static_cast<unsigned>(BH)), block, 0, stream,
                           part_o, part_lse, Hq, S, req_status, out, lse);
    else
        hipLaunchKernelGGL((splitk_combine_wave_kernel<D, 32>), grid, block, 0, stream, part_o, part_lse,
                           BH, Hq, S, req_status, out, lse);
}

}  // namespace

hipError_t launch_splitk_combine(const float *part_o, const float *part_lse, int batch,
                                 int num_q_heads, int num_splits, int head_dim,
                                 const int32_t *req_status, float *out, float *lse,
                                 hipStream_t stream)
{
    const int64_t bh = static_cast<int64_t>(batch) * num_q_heads;
    if (bh > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    const int BH = static_cast<int>(bh);
    if (head_dim == 64)
        launch_combine_wave<64>(part_o, part_lse, BH, num_q_heads, num_splits, req_status, out, lse, stream);
    else if (head_dim == 128)
        launch_combine_wave<128>(part_o, part_lse, BH, num_q_heads, num_splits, req_status, out, lse, stream);
    else
        hipLaunchKernelGGL(splitk_combine_kernel, dim3(static_cast<unsigned>(bh)), dim3(kThreads), 0,
                           stream, part_o, part_lse, num_q_heads, num_splits, head_dim, req_status, out,
                           lse);
    return hipGetLastError();
}

hipError_t launch_bal_combine(const float *part_o, const float *part_lse, const int64_t *prefix,
                              int batch, int num_q_heads, int groups, int head_dim,
                              const int32_t *req_status, const int32_t *context_lens,
                              int max_pages, int log2_page, float *out, float *lse,
                              hipStream_t stream)
{
    const int64_t bh = static_cast<int64_t>(batch) * num_q_heads;
    const int64_t R = static_cast<int64_t>(batch) + groups - 1;
    if (bh > 0x7FFFFFFF || R > 0x7FFFFFFF || (head_dim != 64 && head_dim != 128))
        return hipErrorInvalidConfiguration;
    const unsigned blocks = static_cast<unsigned>((bh + kWaves - 1) / kWaves);
    if (head_dim == 64)
        hipLaunchKernelGGL(bal_combine_wave_kernel<64>, dim3(blocks), dim3(kThreads), 0, stream, part_o,
                           part_lse, prefix, batch, num_q_heads, static_cast<int>(R), req_status,
                           context_lens, max_pages, log2_page, out, lse);
    else
        hipLaunchKernelGGL(bal_combine_wave_kernel<128>, dim3(blocks), dim3(kThreads), 0, stream, part_o,
                           part_lse, prefix, batch, num_q_heads, static_cast<int>(R), req_status,
                           context_lens, max_pages, log2_page, out, lse);
    return hipGetLastError();
}

}  // namespace pafp8
