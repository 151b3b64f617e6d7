// fastdiv.h -- exact unsigned division by a run-time constant as one
// multiply-high, one add and one shift (the round-up method of Granlund and
// Montgomery, "Division by invariant integers using multiplication", PLDI
// 1994, with the 33-bit sum kept in 32 bits by bounding the dividend).
//
// For a divisor d >= 1 let l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1.
// Then for every 0 <= n < 2^31, n / d = (mulhi(n, m) + n) >> l: mulhi(n, m) <= n,
// so the sum stays below 2^32.  Plain C++ (no HIP types), so host code and
// the CPU tests can use the same definition as the kernels.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define TEL_HD __host__ __device__
#else
#define TEL_HD
#endif

namespace tel {

struct FastDiv {
    uint32_t d = 1, m = 1, l = 0;

    FastDiv() = default;
    // d >= 1 and d < 2^31
    explicit FastDiv(uint32_t div) : d(div) {
        l = 0;
        while (l < 31 && (1u << l) < d) ++l;
        m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
    }
    // n / d for 0 <= n < 2^31
    TEL_HD uint32_t div(uint32_t n) const {
#if defined(__HIP_DEVICE_COMPILE__)
        const uint32_t hi = __umulhi(n, m);
#else
        const uint32_t hi = (uint32_t)(((uint64_t)n * m) >> 32);
#endif
        return (hi + n) >> l;
    }
    TEL_HD uint32_t mod(uint32_t n, uint32_t q) const { return n - q * d; }
};

}  // namespace tel
