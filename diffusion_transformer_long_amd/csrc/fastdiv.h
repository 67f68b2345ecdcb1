// Unsigned 32-bit division by a runtime-invariant divisor with one multiply-high,
// after Granlund & Montgomery, "Division by Invariant Integers using Multiplication"
// (PLDI 1994), the round-up variant: with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (t + ((n - t) >> 1)) >> (l - 1) where
// t = mulhi(m, n), for every 32-bit n (d = 1 is special-cased).  Bandwidth-bound index
// math avoids the GPU's long software division sequence this way.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dtl {

struct FastDiv {
    uint32_t d, m, s1, s2;

    __host__ static FastDiv make(uint32_t d) {
        FastDiv f;
        f.d = d;
        if (d == 1) {
            f.m = 0; f.s1 = 0; f.s2 = 0;
            return f;
        }
        uint32_t l = 0;
        while ((1ull << l) < d) ++l;
        f.m = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
        f.s1 = 1;
        f.s2 = l - 1;
        return f;
    }

    __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
        if (d == 1) return n;
        uint32_t t = (uint32_t)(((uint64_t)m * n) >> 32);
        return (t + ((n - t) >> s1)) >> s2;
    }
};

}  // namespace dtl
