// Division by a launch-time constant d >= 1 as a multiply-high, an add and a
// shift: the round-up reciprocal of Granlund and Montgomery ("Division by
// invariant integers using multiplication", 1994) in its "add" form, with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, so that
// q / d = (mulhi(q, m) + q) >> l for every 0 <= q < 2^31.  The kernels use it
// for per-lane index arithmetic, where an integer divide would cost tens of
// VALU instructions.  The host builds the constants; fdiv runs on both sides
// (the CPU test suite checks it against true division exhaustively).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace cnhwc {

struct FastDiv {
    uint32_t mul, shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return FastDiv{uint32_t(m), l};
}

// q in [0, 2^31): mulhi(q, m) <= q, so the add cannot wrap.
__host__ __device__ inline int fdiv(int q, FastDiv f) {
    const uint32_t hi = uint32_t((uint64_t(uint32_t(q)) * f.mul) >> 32);
    return int((hi + uint32_t(q)) >> f.shift);
}

}  // namespace cnhwc
