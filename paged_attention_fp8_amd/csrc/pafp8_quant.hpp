// pafp8_quant.hpp -- the e4m3 encoder and the per-head quantiser used by the
// cache writers and the codec conformance kernel.
//
// The cache format is the pages' "FP8 (e4m3)" (Cloudflare, "Smaller, faster,
// safer: running Kimi and GLM at scale", section "KV 缓存量化"), read as the
// OCP E4M3 encoding: round to nearest even, saturation to +-448, NaN -> S.1111.111.
#pragma once

#include "pafp8_device.hpp"

namespace pafp8 {

// ---------------------------------------------------------------------------
// e4m3 encode: round to nearest even, saturate to +-448, NaN -> 0x7F|sign.
// The hardware conversion rounds to nearest even on the OCP grid; clamping to
// +-448 first turns overflow (and +-inf) into saturation instead of NaN.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e4m3_clamp(float x)
{
    return __builtin_fminf(__builtin_fmaxf(x, -448.0f), 448.0f);  // NaN -> -448, fixed below
}

__device__ __forceinline__ uint32_t e4m3_nan_byte(float x)
{
    return 0x7Fu | ((__float_as_uint(x) >> 24) & 0x80u);
}

// Four values -> four codes packed little-endian (a in the low byte).  NaN
// inputs are rare, so their codes are substituted behind one wave-wide test.
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d)
{
    uint32_t w = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false));
    w = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d),
                                                               static_cast<int>(w), true));
    const bool any_nan = (a != a) | (b != b) | (c != c) | (d != d);
    if (__builtin_amdgcn_ballot_w64(any_nan) != 0) {
        const float v[4] = {a, b, c, d};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (v[i] != v[i])
                w = (w & ~(0xFFu << (8 * i))) | (e4m3_nan_byte(v[i]) << (8 * i));
    }
    return w;
}

__device__ __forceinline__ uint32_t e4m3_encode(float x)
{
    const uint32_t w = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(x), 0.0f, 0, false)) & 0xFFu;
    return x != x ? e4m3_nan_byte(x) : w;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t x) { return __uint_as_float(x << 16); }

// ---------------------------------------------------------------------------
// Quantisation with a per-head scale: code = e4m3(f32(x) / s), the quotient
// rounded as an IEEE single-precision division would round it.
//
// For scales in [2^-64, 2^64] the quotient is formed from the reciprocal and
// one FMA correction (r = 1/s rounded, q0 = |x|*r, e = |x| - q0*s exactly,
// q = q0 + e*r; Markstein's correction step), with |x| first clamped to
// 1024*s (anything larger saturates either way) and the sign copied back.
// An exhaustive comparison with IEEE division over every bf16 significand and
// every fp32 scale significand, plus random signs and exponents over that
// scale range, found no difference; outside the range, or for zero, infinite
// or NaN scales, the kernels divide.
// ---------------------------------------------------------------------------
struct E4m3Quantizer {
    float s, r, lim;
    bool fast;
};

__device__ __forceinline__ E4m3Quantizer make_quantizer(float s)
{
    E4m3Quantizer q;
    q.s = s;
    q.r = 1.0f / s;
    q.lim = 1024.0f * s;
    q.fast = s >= 0x1p-64f && s <= 0x1p64f;
    return q;
}

__device__ __forceinline__ float quotient_fast(float x, const E4m3Quantizer &q)
{
    const float a = __builtin_fminf(__builtin_fabsf(x), q.lim);
    const float q0 = a * q.r;
    const float e = __builtin_fmaf(-q0, q.s, a);
    const float d = __builtin_copysignf(__builtin_fmaf(e, q.r, q0), x);
    return x != x ? x : d;
}

__device__ __forceinline__ uint32_t quantize_bf16(uint16_t x, const E4m3Quantizer &q)
{
    const float xf = bf16_bits_to_f32(x);
    return e4m3_encode(q.fast ? quotient_fast(xf, q) : xf / q.s);
}

// Four bf16 (two dwords, element 0 in the low half of w0) -> four codes.
__device__ __forceinline__ uint32_t quantize_bf16x4(uint32_t w0, uint32_t w1, const E4m3Quantizer &q)
{
    const float x0 = bf16_bits_to_f32(w0 & 0xFFFFu), x1 = bf16_bits_to_f32(w0 >> 16);
    const float x2 = bf16_bits_to_f32(w1 & 0xFFFFu), x3 = bf16_bits_to_f32(w1 >> 16);
    if (q.fast)
        return e4m3_encode4(quotient_fast(x0, q), quotient_fast(x1, q), quotient_fast(x2, q),
                            quotient_fast(x3, q));
    return e4m3_encode4(x0 / q.s, x1 / q.s, x2 / q.s, x3 / q.s);
}

}  // namespace pafp8
