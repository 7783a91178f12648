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

// Wave-per-head combine for the attention's own head dims: one wave owns a
// (request, query head); lane (g, c) handles float4 column c of the splits
// k = g (mod 64 / (D/4)).  The first PF partial rows of every lane are
// loaded together with the split LSEs, so the whole reduction costs one
// memory round trip when S * D <= 64 * 4 * PF.
template <int D>
__global__ __launch_bounds__(kThreads) void splitk_combine_wave_kernel(
    const float *__restrict__ part_o, const float *__restrict__ part_lse, int BH, int Hq, int S,
    const int32_t *__restrict__ req_status, float *__restrict__ out, float *__restrict__ lse_out)
{
    constexpr int NC = D / 4;    // float4 columns of a row
    constexpr int NG = 64 / NC;  // split groups in a wave
    constexpr int PF = 8;        // partial rows per lane loaded up front
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.x * kWaves + uniform(threadIdx.x >> 6);
    if (bh >= BH)
        return;
    const int col = lane % NC, grp = lane / NC;
    const float *pl = part_lse + static_cast<int64_t>(bh) * S;
    const float *po = part_o + static_cast<int64_t>(bh) * S * D + col * 4;
    f32x4 pre[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        const int k = grp + i * NG;
        pre[i] = k < S ? *reinterpret_cast<const f32x4 *>(po + static_cast<int64_t>(k) * D)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float l0 = lane < S ? pl[lane] : kNegInf;
    const bool aborted = req_status != nullptr && req_status[bh / Hq] != 0;
    float M = l0;
    bool nan = l0 != l0;
    for (int k = lane + 64; k < S; k += 64) {
        const float v = pl[k];
        nan |= v != v;
        M = __builtin_fmaxf(M, v);
    }
    M = wave_max(M);
    const bool has_nan = __builtin_amdgcn_ballot_w64(nan) != 0;
    float *o = out + static_cast<int64_t>(bh) * D;
    if (aborted || has_nan || M == kNegInf) {
        const float fill = (has_nan && !aborted) ? __builtin_nanf("") : 0.f;
        if (grp == 0)
            *reinterpret_cast<f32x4 *>(o + col * 4) = f32x4{fill, fill, fill, fill};
        if (lane == 0 && lse_out != nullptr)
            lse_out[bh] = (has_nan && !aborted) ? fill : kNegInf;
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
    if (lane == 0 && lse_out != nullptr)
        lse_out[bh] = LSE;
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
    if (head_dim == 64 || head_dim == 128) {
        const unsigned blocks = static_cast<unsigned>((bh + kWaves - 1) / kWaves);
        if (head_dim == 64)
            hipLaunchKernelGGL(splitk_combine_wave_kernel<64>, dim3(blocks), dim3(kThreads), 0, stream,
                               part_o, part_lse, static_cast<int>(bh), num_q_heads, num_splits,
                               req_status, out, lse);
        else
            hipLaunchKernelGGL(splitk_combine_wave_kernel<128>, dim3(blocks), dim3(kThreads), 0, stream,
                               part_o, part_lse, static_cast<int>(bh), num_q_heads, num_splits,
                               req_status, out, lse);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(splitk_combine_kernel, dim3(static_cast<unsigned>(bh)), dim3(kThreads), 0,
                       stream, part_o, part_lse, num_q_heads, num_splits, head_dim, req_status, out,
                       lse);
    return hipGetLastError();
}

}  // namespace pafp8
