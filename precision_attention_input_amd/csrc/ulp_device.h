// ulp_device.h -- device-side building blocks shared by the libulp kernels (gfx950).
//
// Arithmetic contract (k_grouped_amax page, description: fp32 convert, subtract, abs,
// order-independent max, 1e-7 floor): every float operation is a single IEEE binary32
// operation rounded to nearest-even, fp32 denormals are preserved (the gfx950 default
// float mode), and the library is compiled with -ffp-contract=off so no mul/add pair is
// fused behind our back.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ulp {

constexpr int kGroup = 64;          // rows per global scale group
constexpr float kFloor = 1e-7f;     // amax floor (binary32 nearest to 1e-7)
constexpr int kThreads = 256;       // every kernel runs 256-thread (4-wave) workgroups

enum : int { kBF16 = 0, kFP16 = 1 };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Two packed 16-bit inputs -> two exact binary32 values.
template <int DT>
__device__ __forceinline__ void decode2(uint32_t w, float& lo, float& hi) {
    if constexpr (DT == kBF16) {
        lo = __uint_as_float(w << 16);
        hi = __uint_as_float(w & 0xffff0000u);
    } else {
        half2_t h = __builtin_bit_cast(half2_t, w);
        lo = (float)h.x;
        hi = (float)h.y;
    }
}

// Eight packed 16-bit inputs (one 16-byte vector) -> eight binary32 values.
template <int DT>
__device__ __forceinline__ void decode8(const uint4& v, float* f) {
    decode2<DT>(v.x, f[0], f[1]);
    decode2<DT>(v.y, f[2], f[3]);
    decode2<DT>(v.z, f[4], f[5]);
    decode2<DT>(v.w, f[6], f[7]);
}

template <int DT>
__device__ __forceinline__ float decode1(uint16_t b) {
    if constexpr (DT == kBF16) {
        return __uint_as_float((uint32_t)b << 16);
    } else {
        return (float)__builtin_bit_cast(_Float16, b);
    }
}

__device__ __forceinline__ uint4 load16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ void store16(void* p, const uint4& v) {
    *reinterpret_cast<uint4*>(p) = v;
}

// min(max(x, lo), hi) in one v_med3_f32 for finite lo <= hi.
__device__ __forceinline__ float clampf(float x, float lo, float hi) {
    return __builtin_amdgcn_fmed3f(x, lo, hi);
}

// Max over the lanes of a wave that differ only in the bits of `mask_bits` (xor tree).
template <int OFFSETS_MASK>
__device__ __forceinline__ float wave_max_xor(float v) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
        if (OFFSETS_MASK & off) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

template <int OFFSETS_MASK>
__device__ __forceinline__ float wave_min_xor(float v) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
        if (OFFSETS_MASK & off) v = fminf(v, __shfl_xor(v, off, 64));
    return v;
}

// ---------------------------------------------------------------- INT8 quantization
//
// code = clamp(rint(RN(x / s)), -127, 127) with RN(x / s) the IEEE quotient.
//
// Fast path: with y = RN(1/s), t = RN(x * y) satisfies |t - RN(x/s)| <= (3u + u^2)/(1-2u-u^2)
// |t| < 2^-21 |t| (u = 2^-24): y carries relative error <= u, the product adds <= u, and
// RN(x/s) is within u of x/s.  So whenever t lies farther than 2^-21 |t| from every
// half-integer, RN(x/s) lies strictly on the same side of every half-integer as t and
// rint gives the same integer.  Only the rare t close to a half-integer needs the true
// quotient.  Quotients are first clamped to [-128, 128]; every value beyond rounds and
// clamps to +-127 either way.
struct QuantScale {
    float s;   // the stored fp32 scale
    float y;   // RN(1 / s)
};

__device__ __forceinline__ QuantScale make_scale(float amax) {
    QuantScale q;
    q.s = amax / 127.0f;     // IEEE division (correctly rounded)
    q.y = 1.0f / q.s;
    return q;
}

// Quantize N values; returns the rounded (not yet clamped to +-127) quotients in r.
template <int N>
__device__ __forceinline__ void quantize_n(const float* x, const QuantScale& qs, float* r) {
    bool near = false;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float t = clampf(x[i] * qs.y, -128.0f, 128.0f);
        r[i] = __builtin_rintf(t);
        near |= (__builtin_fabsf(t - r[i]) + __builtin_fabsf(t) * 0x1p-21f) >= 0.5f;
    }
    if (__builtin_expect(near, 0)) {
#pragma unroll
        for (int i = 0; i < N; ++i) r[i] = __builtin_rintf(clampf(x[i] / qs.s, -128.0f, 128.0f));
    }
}

// Four rounded quotients -> four int8 codes packed little-endian in a dword.
__device__ __forceinline__ uint32_t pack_i8x4(float a, float b, float c, float d) {
    uint32_t ia = (uint32_t)(int)clampf(a, -127.0f, 127.0f);
    uint32_t ib = (uint32_t)(int)clampf(b, -127.0f, 127.0f);
    uint32_t ic = (uint32_t)(int)clampf(c, -127.0f, 127.0f);
    uint32_t id = (uint32_t)(int)clampf(d, -127.0f, 127.0f);
    // byte 0 of each: selector 0x0c yields a zero byte
    uint32_t lo = __builtin_amdgcn_perm(ib, ia, 0x0c0c0400u);   // [a0, b0, 0, 0]
    uint32_t hi = __builtin_amdgcn_perm(id, ic, 0x04000c0cu);   // [0, 0, c0, d0]
    return lo | hi;
}

// ---------------------------------------------------------------- FP8 E4M3 (OCP E4M3FN)
//
// gfx950's v_cvt_pk_fp8_f32 converts to OCP E4M3FN with round-to-nearest-even.  Inputs are
// clamped to +-448 first, so every finite input saturates to the largest finite code
// instead of reaching the NaN pattern.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    a = clampf(a, -448.0f, 448.0f);
    b = clampf(b, -448.0f, 448.0f);
    c = clampf(c, -448.0f, 448.0f);
    d = clampf(d, -448.0f, 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// ---------------------------------------------------------------- 4x4 byte transpose
//
// rows a, b, c, d (little-endian dwords, byte k = column k) -> columns c0..c3 where column
// k holds [a.k, b.k, c.k, d.k].
__device__ __forceinline__ void transpose4x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                             uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                             uint32_t& c3) {
    uint32_t t0 = __builtin_amdgcn_perm(b, a, 0x05010400u);   // [a0, b0, a1, b1]
    uint32_t t1 = __builtin_amdgcn_perm(b, a, 0x07030602u);   // [a2, b2, a3, b3]
    uint32_t t2 = __builtin_amdgcn_perm(d, c, 0x05010400u);   // [c0, d0, c1, d1]
    uint32_t t3 = __builtin_amdgcn_perm(d, c, 0x07030602u);   // [c2, d2, c3, d3]
    c0 = __builtin_amdgcn_perm(t2, t0, 0x05040100u);          // [a0, b0, c0, d0]
    c1 = __builtin_amdgcn_perm(t2, t0, 0x07060302u);          // [a1, b1, c1, d1]
    c2 = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    c3 = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// ---------------------------------------------------------------- geometry
__device__ __forceinline__ int64_t first_group(int64_t r, int64_t L) { return r * L / kGroup; }
__device__ __forceinline__ int64_t last_group(int64_t r, int64_t L) {
    return (r * L + L - 1) / kGroup;
}

}  // namespace ulp
