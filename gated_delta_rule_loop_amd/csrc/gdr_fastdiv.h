// Division by a divisor fixed for a launch, as a multiply and a shift (host
// side; the kernels apply the formula).  Part of the library's internals,
// not of the public ABI; free of HIP so that host tests can include it.
#pragma once

#include <stdint.h>

namespace gdr {

// x / d for every non-negative x below 2^31 and 1 <= d < 2^31:
//   q = (mulhi(x, mul) + x) >> shift,
// shift = ceil(log2 d), mul = floor(2^32 (2^shift - d) / d) + 1.  mulhi(x,
// mul) < x, so the sum stays below 2^32.
struct FastDiv {
    uint32_t mul, shift;
};
inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t s = 0;
    while ((uint64_t{1} << s) < d) ++s;
    const uint64_t m = ((uint64_t{1} << 32) * ((uint64_t{1} << s) - d)) / d + 1;
    return FastDiv{static_cast<uint32_t>(m), s};
}

}  // namespace gdr
