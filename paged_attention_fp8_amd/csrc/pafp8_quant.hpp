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
// one FMA correction (Markstein's step: r = 1/s rounded, q0 = x*r rounded,
// t = q0*s - x exactly, q = q0 - t*r), after clamping x to +-c, c = 440*s
// rounded.  Every |x| >= c lies above 432*s, where the code is the one of 448
// whatever the exact quotient, and the clamped quotient never exceeds 448, so
// the conversion needs no clamp of its own.  Forming the remainder as
// q0*s - x and subtracting it keeps the sign of a zero quotient.
//
// Any other finite non-zero scale (negative ones included) is first written
// as |s| = m 2^e with m in [1, 2); x / s equals ldexp(+-x, -e) / m exactly
// unless the rescaled x overflows (then the code saturates either way) or
// underflows (then the quotient is below 2^-126 and its code is a zero of
// the right sign either way), and the same steps run on the rescaled pair.
// Zero, infinite and NaN scales give unspecified codes.
//
// An exhaustive CPU comparison with IEEE division (every bf16 significand of
// both signs against every fp32 scale significand, every value of the clamp
// region, random values against random scales over the range and, rescaled,
// outside it) found no difference in the quotient where no clamp acts and
// none in the code anywhere.  NaN inputs are patched afterwards
// (e4m3_nan_byte).
// ---------------------------------------------------------------------------
struct E4m3Quantizer {
    float s, r, lim;   // divisor (the scale, or m), its reciprocal, the clamp
    int shift;         // exponent added to x before dividing (rescaled form)
    uint32_t sign;     // sign bit flipped on x (rescaled form, negative scales)
    bool fast;         // s in [2^-64, 2^64]: no rescaling
};

__device__ __forceinline__ E4m3Quantizer make_quantizer(float s)
{
    E4m3Quantizer q;
    q.fast = s >= 0x1p-64f && s <= 0x1p64f;
    q.shift = 0;
    q.sign = 0u;
    q.s = s;
    if (!q.fast) {
        const float a = __builtin_fabsf(s);
        q.s = 2.0f * __builtin_amdgcn_frexp_mantf(a);          // [1, 2) for finite non-zero s
        q.shift = 1 - __builtin_amdgcn_frexp_expf(a);
        q.sign = __float_as_uint(s) & 0x80000000u;
    }
    q.r = 1.0f / q.s;
    q.lim = 440.0f * q.s;
    return q;
}

// the quotient, ready for the conversion (|result| <= 448 unless x is NaN)
template <bool FAST>
__device__ __forceinline__ float quotient(float x, const E4m3Quantizer &q)
{
    if constexpr (!FAST)
        x = __builtin_amdgcn_ldexpf(__uint_as_float(__float_as_uint(x) ^ q.sign), q.shift);
    const float xc = __builtin_amdgcn_fmed3f(x, -q.lim, q.lim);
    const float q0 = xc * q.r;
    const float t = __builtin_fmaf(q0, q.s, -xc);
    return __builtin_fmaf(-t, q.r, q0);
}

// two quotients -> two codes in half HI of w (the other half kept)
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b, uint32_t w)
{
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, static_cast<int>(w), HI));
}

// byte i of w replaced by the NaN code of x when x is NaN
__device__ __forceinline__ uint32_t e4m3_patch_nan(uint32_t w, int i, float x)
{
    return x != x ? (w & ~(0xFFu << (8 * i))) | (e4m3_nan_byte(x) << (8 * i)) : w;
}

__device__ __forceinline__ uint32_t quantize_bf16(uint16_t x, const E4m3Quantizer &q)
{
    const float xf = bf16_bits_to_f32(x);
    const float v = q.fast ? quotient<true>(xf, q) : quotient<false>(xf, q);
    const uint32_t w = e4m3_pack2<false>(v, 0.0f, 0u) & 0xFFu;
    return xf != xf ? e4m3_nan_byte(xf) : w;
}

}  // namespace pafp8
