// pafp8_device.hpp -- device-side building blocks for gfx950 (CDNA4).
//
// The e4m3 decode routes the attention kernels use, the MFMA operand types,
// 16-byte global loads, and small wave helpers (the encoder and quantiser are
// in pafp8_quant.hpp).  The cache format is the pages' "FP8 (e4m3)"
// (Cloudflare, "Smaller, faster, safer: running Kimi and GLM at scale",
// section "KV 缓存量化" / KV cache quantization), read as the OCP E4M3 encoding
// (bias 7, no infinities, +-448 largest finite value), which gfx950's
// conversion instructions implement.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pafp8 {

typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef _Float16 f16x2 __attribute__((__vector_size__(2 * sizeof(_Float16))));
typedef float f32x2 __attribute__((__vector_size__(2 * sizeof(float))));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// e4m3 decode routes.  Every e4m3 value is exact in fp16, bf16 and fp32.
// ---------------------------------------------------------------------------
// 4 codes (one dword) -> 2 packed bf16 pairs, exact (scale 1.0 = identity).
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w)
{
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    u32x2 r;
    r[0] = __builtin_bit_cast(uint32_t, lo);
    r[1] = __builtin_bit_cast(uint32_t, hi);
    return r;
}

// 4 codes -> 2 packed fp16 pairs, exact.
__device__ __forceinline__ u32x2 e4m3x4_to_f16x4(uint32_t w)
{
    const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
    u32x2 r;
    r[0] = __builtin_bit_cast(uint32_t, lo);
    r[1] = __builtin_bit_cast(uint32_t, hi);
    return r;
}

// 8 codes (two dwords) -> an 8-element MFMA operand.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1)
{
    const u32x2 a = e4m3x4_to_bf16x4(w0);
    const u32x2 b = e4m3x4_to_bf16x4(w1);
    u32x4 r = {a[0], a[1], b[0], b[1]};
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ f16x8 e4m3x8_to_f16x8(uint32_t w0, uint32_t w1)
{
    const u32x2 a = e4m3x4_to_f16x4(w0);
    const u32x2 b = e4m3x4_to_f16x4(w1);
    u32x4 r = {a[0], a[1], b[0], b[1]};
    return __builtin_bit_cast(f16x8, r);
}

// 2 codes (the low or high half of a dword) -> 2 fp32, exact.
template <bool HIGH_HALF>
__device__ __forceinline__ f32x2 e4m3x2_to_f32x2(uint32_t w)
{
    return __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), HIGH_HALF);
}

// ---------------------------------------------------------------------------
// packing fp32 -> 16-bit MFMA operands (round to nearest even)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b)
{
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// memory
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 load16(const void *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

// Data read exactly once per call (KV, weights): stream it past the caches.
__device__ __forceinline__ u32x4 load16_stream(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ void store16(void *p, u32x4 v)
{
    *reinterpret_cast<u32x4 *>(p) = v;
}

// ---------------------------------------------------------------------------
// MFMA: D(16x16 fp32) += A(16x32) * B(32x16).  Lane l supplies A[l%16][k]
// and B[k][l%16] for the eight k of group l/16, and holds D rows
// 4*(l/16)+0..3 of column l%16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// wave helpers (wave64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor_f(float v, int mask)
{
    return __shfl_xor(v, mask, 64);
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v = __builtin_fmaxf(v, shfl_xor_f(v, m));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += shfl_xor_f(v, m);
    return v;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace pafp8
