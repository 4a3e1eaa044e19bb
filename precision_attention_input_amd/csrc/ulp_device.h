// ulp_device.h -- device-side building blocks shared by the libulp kernels (gfx950).
//
// Arithmetic contract (k_grouped_amax page, description): inputs are widened to binary32,
// centered and taken in magnitude, the group maximum does not depend on the order of the
// rows, and the result never drops below the 1e-7 floor.  Every float operation is a
// single IEEE binary32 operation rounded to nearest-even, fp32 denormals are preserved (the gfx950 default
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

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte global accesses.  NT = true marks the access non-temporal (streamed, not kept in
// the caches); each launcher picks the policy from the size of its streams (see below).
template <bool NT = false>
__device__ __forceinline__ uint4 load16(const void* p) {
    if constexpr (NT) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *reinterpret_cast<const uint4*>(p);
    }
}

template <bool NT = false>
__device__ __forceinline__ void store16(void* p, const uint4& v) {
    if constexpr (NT) {
        const u32x4_t w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
    } else {
        *reinterpret_cast<uint4*>(p) = v;
    }
}

// Cache policy.  A stream whose bytes fit comfortably in the 256 MB last-level cache
// (Infinity Cache) is read and written with the default policy, so the next kernel of the
// step finds it there (the pack re-reads Q and K right after the statistics pass; the
// unpack reads the chunks the pack just wrote).  Larger streams cannot stay resident, and
// non-temporal accesses then keep them from evicting data that can; the launchers pick the
// instantiation from the stream's size.  The unpack's outputs, which nothing in the path
// reads again, are always streamed.
#ifndef ULP_RESIDENT_MB
#define ULP_RESIDENT_MB 128
#endif
constexpr int64_t kResidentBytes = (int64_t)ULP_RESIDENT_MB << 20;


// min(max(x, lo), hi) in one v_med3_f32 for finite lo <= hi.
__device__ __forceinline__ float clampf(float x, float lo, float hi) {
    return __builtin_amdgcn_fmed3f(x, lo, hi);
}

// Max / min over the lanes of a wave that differ only in the bits of OFFSETS_MASK, left in
// every such lane.  No LDS traffic: inside a 16-lane row the lanes are combined with DPP
// (row_mirror pairs lane i with 15 - i, row_half_mirror i with 7 - i inside each 8, then the
// quad permutations [2,3,0,1] and [1,0,3,2]: after these every lane has met its whole row,
// or its whole half-row when only bits 0-2 are asked for; bit 3 alone is a rotation of the
// row by 8); bits 4 and 5 use gfx950's
// v_permlane16_swap / v_permlane32_swap on two copies of the value.  Other bit patterns
// fall back to LDS lane permutes.  Max and min are order-independent, so every lane ends
// with the same bits.
template <bool MAX>
__device__ __forceinline__ float pick(float a, float b) {
    return MAX ? fmaxf(a, b) : fminf(a, b);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <bool MAX, int OFFSETS_MASK>
__device__ __forceinline__ float wave_reduce_xor(float v) {
    constexpr int low = OFFSETS_MASK & 15;
    if constexpr (low == 15) {
        v = pick<MAX>(v, dpp<0x140>(v));        // row_mirror
        v = pick<MAX>(v, dpp<0x141>(v));        // row_half_mirror
        v = pick<MAX>(v, dpp<0x4E>(v));         // quad_perm [2,3,0,1]
        v = pick<MAX>(v, dpp<0xB1>(v));         // quad_perm [1,0,3,2]
    } else if constexpr (low == 7) {
        v = pick<MAX>(v, dpp<0x141>(v));
        v = pick<MAX>(v, dpp<0x4E>(v));
        v = pick<MAX>(v, dpp<0xB1>(v));
    } else if constexpr (low == 8) {
        v = pick<MAX>(v, dpp<0x128>(v));        // row_ror 8: lane i meets lane i ^ 8
    } else {
#pragma unroll
        for (int off = 1; off < 16; off <<= 1)
            if (low & off) v = pick<MAX>(v, __shfl_xor(v, off, 64));
    }
    if constexpr ((OFFSETS_MASK & 16) != 0) {
        const unsigned u = __float_as_uint(v);
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        v = pick<MAX>(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    if constexpr ((OFFSETS_MASK & 32) != 0) {
        const unsigned u = __float_as_uint(v);
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        v = pick<MAX>(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    return v;
}

template <int OFFSETS_MASK>
__device__ __forceinline__ float wave_max_xor(float v) {
    return wave_reduce_xor<true, OFFSETS_MASK>(v);
}

template <int OFFSETS_MASK>
__device__ __forceinline__ float wave_min_xor(float v) {
    return wave_reduce_xor<false, OFFSETS_MASK>(v);
}

// ---------------------------------------------------------------- INT8 quantization
//
// code = clamp(rint(RN(x / s)), -127, 127) with RN(x / s) the IEEE quotient.
//
// Fast path: t = RN(x * y) with y the hardware reciprocal of s.  v_rcp_f32 is within 1 ulp
// of the correctly rounded reciprocal (checked on gfx950 for every mantissa), so with
// u = 2^-24, |y - 1/s| <= 1.5 ulp <= 3u/s.  Then |x*y - x/s| <= 3u|x/s|, the product's
// rounding adds <= u(1+3u)|x/s|, and RN(x/s) is within u|x/s| of x/s, so
//   |t - RN(x/s)| <= (5u + 3u^2) |x/s| <= (5u + 3u^2) / (1 - 4u - 3u^2) |t| < 2^-21 |t|.
// Whenever t lies farther than 2^-21 |t| from every half-integer, RN(x/s) lies strictly on
// the same side of every half-integer as t and rint gives the same integer.  Only the rare
// t close to a half-integer needs the true quotient (checked per 16 values, fixed after the
// fast-path codes are stored).
//
// Clamping the quotient to [-127, 127] before rint is the same as clamping the rounded
// integer afterwards (the bounds are integers and rint is monotone), and a clamped t sits
// exactly on an integer, so the near-half-integer test never fires for it.  The test is
// |t - rint(t)| + 2^-21 |t| >= 1/2, one fma per value (the product by 2^-21 is exact).
struct QuantScale {
    float s;     // the stored fp32 scale, RN(amax / 127)
    float y;     // reciprocal of s within 1 ulp
    float s24;   // s * 2^-24 (exact)
};

__device__ __forceinline__ QuantScale make_scale(float amax) {
    QuantScale q;
    q.s = amax / 127.0f;                     // IEEE division (correctly rounded)
    q.y = __builtin_amdgcn_rcpf(q.s);        // s >= 1e-7/127 is normal: no denormal issue
    q.s24 = q.s * 0x1p-24f;
    return q;
}

// Fast path over N values: int8 codes (as int) in c; returns the largest
// |t - rint(t)| + 2^-21 |t| (>= 0.5 means some value needs the exact decision).
template <int N>
__device__ __forceinline__ float quantize_fast(const float* x, const QuantScale& qs, int* c) {
    float worst = 0.0f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float t = clampf(x[i] * qs.y, -127.0f, 127.0f);
        const float r = __builtin_rintf(t);
        c[i] = (int)r;
        worst = fmaxf(worst, __builtin_fmaf(__builtin_fabsf(t), 0x1p-21f, __builtin_fabsf(t - r)));
    }
    return worst;
}

// Exact decision without a division: clamp(rint(RN(x/s)), -127, 127) for any x.
//
// Let k = floor(t) for t = x*y clamped to [-127.25, 127.25], and h = k + 1/2.  Because t is
// within 2^-21 |t| of RN(x/s), rint(RN(x/s)) is k if RN(x/s) < h, k+1 if RN(x/s) > h, and
// the even one of the two if RN(x/s) == h (values clamped at +-127.25 end at +-127 in every
// case).  h has at most 9 significant bits, so its last significand bit is 0: its float
// neighbours are h -+ 2e with e = ulp(h)/2, and a quotient exactly on a midpoint h -+ e rounds
// to h.  (For |h| = 1/2 the midpoint toward zero is at e/2, but there both outcomes on that
// side give the same code, 0.)  So RN(x/s) == h  <=>  |x - s*h| <= s*e, and the sign of
// x - s*h orders x/s against h.  D = fma(-s, h, x) is x - s*h exactly whenever |x - s*h| is
// near s*e: x and s*h are then multiples of a common power of two at most 2^13 times smaller
// than |D|, so D needs at most 13 significant bits; elsewhere D still has the right sign and
// lies far from +-s*e.  s*e = (s * 2^-24) * 2^exponent(h) is exact.
template <int N>
__device__ __forceinline__ void quantize_exact(const float* x, const QuantScale& qs, int* c) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float t = clampf(x[i] * qs.y, -127.25f, 127.25f);
        const float k = __builtin_floorf(t);
        const float h = k + 0.5f;
        const float d = __builtin_fmaf(-qs.s, h, x[i]);
        const float e = qs.s24 * __uint_as_float(__float_as_uint(h) & 0x7f800000u);
        const int ki = (int)k;
        const int inc = d > e ? 1 : (__builtin_fabsf(d) <= e ? (ki & 1) : 0);
        c[i] = min(max(ki + inc, -127), 127);
    }
}

template <int N>
__device__ __forceinline__ void quantize_n(const float* x, const QuantScale& qs, int* c) {
    if (__builtin_expect(!(quantize_fast<N>(x, qs, c) < 0.5f), 0)) quantize_exact<N>(x, qs, c);
}

// Four int8 codes (held as int in [-127, 127]) packed little-endian in a dword.
__device__ __forceinline__ uint32_t pack_i8x4(int a, int b, int c, int d) {
    const uint32_t ia = (uint32_t)a, ib = (uint32_t)b, ic = (uint32_t)c, id = (uint32_t)d;
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
