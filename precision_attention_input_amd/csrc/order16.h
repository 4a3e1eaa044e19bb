// order16.h -- order statistics of 16-bit floats on their raw bit patterns (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ulp {

// Order statistics of 16-bit floats (bf16 or fp16) without converting them.  Both formats
// are sign-magnitude with the sign in bit 15.  Read as signed integers, the non-negative
// values keep their order and sort above every negative one; read as unsigned integers,
// the non-negative values keep their order and sort below every negative one, and the
// negative ones sort by magnitude.  So over a set of non-NaN values
//   max = smax(set) if that is non-negative (sign bit clear), else umin(set);
//   min = umax(set) if that is negative (sign bit set),       else umin(set),
// with smax / umin / umax the signed maximum, unsigned minimum and unsigned maximum of the
// bit patterns: three packed 16-bit integer operations per two values.  -0 and +0 may come
// out either way round; callers canonicalise zeros.
typedef short i16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

struct Order16 {
    uint32_t smax, umin, umax;   // two values per word

    __device__ __forceinline__ void reset() {
        smax = 0x80008000u;      // smallest signed, largest and smallest unsigned patterns
        umin = 0xffffffffu;
        umax = 0u;
    }
    __device__ __forceinline__ void add(uint32_t w) {
        const i16x2_t sw = __builtin_bit_cast(i16x2_t, w);
        const u16x2_t uw = __builtin_bit_cast(u16x2_t, w);
        smax = __builtin_bit_cast(uint32_t,
                                  __builtin_elementwise_max(__builtin_bit_cast(i16x2_t, smax), sw));
        umin = __builtin_bit_cast(uint32_t,
                                  __builtin_elementwise_min(__builtin_bit_cast(u16x2_t, umin), uw));
        umax = __builtin_bit_cast(uint32_t,
                                  __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, umax), uw));
    }
    // The two maxima / minima as packed 16-bit patterns (meaningful after at least one add).
    __device__ __forceinline__ uint32_t max_bits() const {
        const uint32_t neg = __builtin_bit_cast(
            uint32_t, __builtin_bit_cast(i16x2_t, smax) >> (i16x2_t){15, 15});
        return (umin & neg) | (smax & ~neg);
    }
    __device__ __forceinline__ uint32_t min_bits() const {
        const uint32_t neg = __builtin_bit_cast(
            uint32_t, __builtin_bit_cast(i16x2_t, umax) >> (i16x2_t){15, 15});
        return (umax & neg) | (umin & ~neg);
    }
};

// Order16 of two partial sets -> Order16 of their union.
__device__ __forceinline__ Order16 merge(const Order16& a, const Order16& b) {
    Order16 r;
    r.smax = __builtin_bit_cast(uint32_t,
                                __builtin_elementwise_max(__builtin_bit_cast(i16x2_t, a.smax),
                                                          __builtin_bit_cast(i16x2_t, b.smax)));
    r.umin = __builtin_bit_cast(uint32_t,
                                __builtin_elementwise_min(__builtin_bit_cast(u16x2_t, a.umin),
                                                          __builtin_bit_cast(u16x2_t, b.umin)));
    r.umax = __builtin_bit_cast(uint32_t,
                                __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a.umax),
                                                          __builtin_bit_cast(u16x2_t, b.umax)));
    return r;
}

}  // namespace ulp
