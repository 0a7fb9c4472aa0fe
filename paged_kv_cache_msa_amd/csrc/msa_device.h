// Device arithmetic shared by the producer kernels (fused and unfused): bf16 unpacking, the
// bf16 and OCP FP8 E4M3 output casts, the RMSNorm scale, the RoPE coefficients and the 8-lane
// head reduction.  Both producers take every rounding from these functions, so their outputs are
// the same bytes.  Internal to the library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "msa_common.h"

namespace msa_internal {

constexpr int kHalf = kHeadDim / 2;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const uint4& v, float* f)
{
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two binary32 -> bf16 round-to-nearest-even (v_cvt_pk_bf16_f32); NaN -> quiet NaN, sign kept.
__device__ __forceinline__ uint32_t bf16x2(float a, float b)
{
    f32x2_t v = {a, b};
    bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
    uint32_t w;
    __builtin_memcpy(&w, &h, 4);
    return w;
}

__device__ __forceinline__ float sat448(float v) { return fabsf(v) > 448.0f ? copysignf(448.0f, v) : v; }

// Four binary32 -> OCP E4M3, round-to-nearest-even, saturating to +-448 (infinities included).
// v_cvt_pk_fp8_f32 rounds to nearest even but does not saturate and writes 0xff for every NaN;
// the clamp runs first (a NaN fails the compare and passes through) and positive NaNs get their
// sign bit cleared afterwards so that a NaN keeps its sign.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d)
{
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), w, true);
    uint32_t clear = (__float_as_int(a) > 0x7f800000 ? 0x80u : 0u) | (__float_as_int(b) > 0x7f800000 ? 0x8000u : 0u)
                   | (__float_as_int(c) > 0x7f800000 ? 0x800000u : 0u) | (__float_as_int(d) > 0x7f800000 ? 0x80000000u : 0u);
    return w & ~clear;
}

// Four binary32 -> E4M3 with the conversion instruction alone: round-to-nearest-even, equal to
// e4m3x4 wherever no byte comes out as a NaN code (a NaN input, or a magnitude of 464 or more:
// the instruction writes a NaN code there instead of saturating).
__device__ __forceinline__ uint32_t e4m3x4_rne(float a, float b, float c, float d)
{
    const uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Nonzero iff some byte of w is an E4M3 NaN code (its low seven bits all set): adding 1 to the
// low seven bits of each byte carries into bit 7 exactly there, never into the next byte.
__device__ __forceinline__ uint32_t e4m3_nan_bytes(uint32_t w)
{
    return ((w & 0x7f7f7f7fu) + 0x01010101u) & 0x80808080u;
}

// Dequantisation scale -> quantisation multiplier, binary32 division rounded once.
__device__ __forceinline__ float inv_scale(float scale) { return 1.0f / scale; }
__device__ __forceinline__ float inv_scale_of(const float* scale) { return inv_scale(*scale); }

// RMSNorm scale from a binary64 sum of squares: (float)(1 / sqrt(ss / 128 + eps)).
__device__ __forceinline__ float rms_from_ss(double ss, float eps)
{
    return (float)(1.0 / sqrt(ss / (double)kHeadDim + (double)eps));
}

// RoPE coefficient pair of one (position, frequency).
__device__ __forceinline__ void rope_coeff(int32_t pos, double inv_freq, float* c, float* s)
{
    const double angle = (double)pos * inv_freq;
    double sn, cs;
    sincos(angle, &sn, &cs);
    *c = (float)cs;
    *s = (float)sn;
}

template <int Ctrl>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, Ctrl, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), Ctrl, 0xf, 0xf, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Sum over the 8 lanes of a head.  Every lane of the group ends with the same value: each step
// adds a partner's partial, and IEEE addition is commutative.
__device__ __forceinline__ double head_sum8(double v)
{
    v += dpp_f64<0xb1>(v);    // quad_perm [1,0,3,2]: partner lane ^ 1
    v += dpp_f64<0x4e>(v);    // quad_perm [2,3,0,1]: partner lane ^ 2
    v += dpp_f64<0x141>(v);   // row_half_mirror: lane i <- 7 - i within each group of 8
    return v;
}


typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Output stores.  Streaming (nontemporal) stores keep large batches' write-once outputs from
// displacing cache lines still to be read; small batches use ordinary stores so that their
// consumer (the next kernel) finds Q and the new cache rows in cache.
template <bool kStream>
__device__ __forceinline__ void store16(void* p, uint4 v)
{
    if (kStream) {
        const u32x4_t w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
    } else {
        *reinterpret_cast<uint4*>(p) = v;
    }
}

// Input row loads: nontemporal for large batches (each row is read once).
template <bool kStream>
__device__ __forceinline__ uint4 load16(const void* p)
{
    if (kStream) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
        return make_uint4(v[0], v[1], v[2], v[3]);
    }
    return *reinterpret_cast<const uint4*>(p);
}

template <bool kStream>
__device__ __forceinline__ void store8(void* p, uint2 v)
{
    if (kStream) {
        const u32x2_t w = {v.x, v.y};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(p));
    } else {
        *reinterpret_cast<uint2*>(p) = v;
    }
}

// Per-lane fp8 cast of 16 values (scaled by m) into two 8-byte halves.  When no value of the lane
// needs saturation or NaN handling (|v| <= 448), the bare hardware conversion already is the exact
// saturating RNE cast; otherwise the full cast runs.
__device__ __forceinline__ void e4m3x16(const float* o, float m, uint2& lo, uint2& hi)
{
    float z[16];
    uint32_t a[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        z[j] = o[j] * m;
        a[j] = __float_as_uint(z[j]) & 0x7fffffffu;   // |z| as bits: ordered like |z|, NaN above infinity
    }
    // Largest magnitude by a balanced tree (4 dependent steps instead of a 16-long chain of tests):
    // special iff some |z| > 448, an infinity or a NaN.
#pragma unroll
    for (int w = 8; w >= 1; w /= 2)
#pragma unroll
        for (int j = 0; j < w; ++j) a[j] = a[j] > a[j + w] ? a[j] : a[j + w];
    const bool special = a[0] > 0x43e00000u;           // bits of 448.0f
    uint32_t w[4];
    if (!special) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t l = __builtin_amdgcn_cvt_pk_fp8_f32(z[4 * q], z[4 * q + 1], 0, false);
            w[q] = __builtin_amdgcn_cvt_pk_fp8_f32(z[4 * q + 2], z[4 * q + 3], l, true);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = e4m3x4(z[4 * q], z[4 * q + 1], z[4 * q + 2], z[4 * q + 3]);
    }
    lo = make_uint2(w[0], w[1]);
    hi = make_uint2(w[2], w[3]);
}

__device__ __forceinline__ uint4 bf16x8(const float* o)
{
    return make_uint4(bf16x2(o[0], o[1]), bf16x2(o[2], o[3]), bf16x2(o[4], o[5]), bf16x2(o[6], o[7]));
}

}  // namespace msa_internal
