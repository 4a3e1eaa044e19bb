// pack_device.h -- per-vector quantization shared by the pack kernels (gfx950).
//
// Sixteen consecutive channels of one row, held as two raw 16-byte words, become sixteen
// INT8 codes (Q raw, K centered on the mean; one 16-byte word of codes) or sixteen E4M3
// bytes (V): the element formulas of the pack step that the k_grouped_amax page
// (description) feeds, with the scale arithmetic of ulp_device.h.
#pragma once

#include "ulp_device.h"

namespace ulp {

template <int DT>
__device__ __forceinline__ void decode16(const uint4& a, const uint4& b, float* f) {
    decode8<DT>(a, f);
    decode8<DT>(b, f + 8);
}

__device__ __forceinline__ uint4 codes16(const int* c) {
    return make_uint4(pack_i8x4(c[0], c[1], c[2], c[3]), pack_i8x4(c[4], c[5], c[6], c[7]),
                      pack_i8x4(c[8], c[9], c[10], c[11]),
                      pack_i8x4(c[12], c[13], c[14], c[15]));
}

// 16 inputs held as two raw 16-byte words (K: minus the mean, also two raw words) -> fp32.
template <int DT, bool CENTER>
__device__ __forceinline__ void inputs16(const uint4& a, const uint4& b, const uint4& ma,
                                         const uint4& mb, float* f) {
    decode16<DT>(a, b, f);
    if constexpr (CENTER) {
        float m[16];
        decode16<DT>(ma, mb, m);
#pragma unroll
        for (int e = 0; e < 16; ++e) f[e] = f[e] - m[e];
    }
}

// Codes of 16 inputs.  EXACT_ONLY: the division-free exact decision for every value.
// Otherwise the fast path, falling back to the exact decision when any value of the
// wave's vectors lies near a half-integer (re-decoding from the raw words keeps few
// registers live across the fast path).  The exact decision costs about twice the fast
// path, so it pays to skip the fast path where near-ties are the rule: centered K (small
// deviations on a coarse grid) and bf16 Q (8-bit significands): the kernels instantiate
// EXACT_ONLY for those two and the fast path for fp16 Q.
template <int DT, bool CENTER, bool EXACT_ONLY>
__device__ __forceinline__ uint4 quantize16(const uint4& a, const uint4& b, const uint4& ma,
                                            const uint4& mb, const QuantScale& sc) {
    float f[16];
    int c[16];
    inputs16<DT, CENTER>(a, b, ma, mb, f);
    if constexpr (EXACT_ONLY) {
        quantize_exact<16>(f, sc, c);
    } else if (__builtin_expect(!(quantize_fast<16>(f, sc, c) < 0.5f), 0)) {
        inputs16<DT, CENTER>(a, b, ma, mb, f);
        quantize_exact<16>(f, sc, c);
    }
    return codes16(c);
}

template <int DT>
__device__ __forceinline__ uint4 e4m3x16(const uint4& x0, const uint4& x1) {
    float f[16];
    decode16<DT>(x0, x1, f);
    return make_uint4(e4m3x4(f[0], f[1], f[2], f[3]), e4m3x4(f[4], f[5], f[6], f[7]),
                      e4m3x4(f[8], f[9], f[10], f[11]), e4m3x4(f[12], f[13], f[14], f[15]));
}

// V divided by the caller's scale (one correctly rounded binary32 division per value: the
// compiler's default single-precision division on gfx950), then E4M3.
template <int DT>
__device__ __forceinline__ uint4 e4m3x16_scaled(const uint4& x0, const uint4& x1,
                                                const float4* sv) {
    float f[16];
    decode16<DT>(x0, x1, f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[4 * i] = f[4 * i] / sv[i].x;
        f[4 * i + 1] = f[4 * i + 1] / sv[i].y;
        f[4 * i + 2] = f[4 * i + 2] / sv[i].z;
        f[4 * i + 3] = f[4 * i + 3] / sv[i].w;
    }
    return make_uint4(e4m3x4(f[0], f[1], f[2], f[3]), e4m3x4(f[4], f[5], f[6], f[7]),
                      e4m3x4(f[8], f[9], f[10], f[11]), e4m3x4(f[12], f[13], f[14], f[15]));
}

}  // namespace ulp
