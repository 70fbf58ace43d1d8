// Exhaustive CPU check of the library's division by launch constants
// (convolution_nhwc_amd/csrc/fastdiv.h): make_fastdiv's constants and fdiv's
// multiply-high, add and shift, the same inline functions the kernels call,
// against true integer division.
//
//   every divisor 1..70000   x  every dividend 0..2^20-1
//   every divisor 1..70000   x  dividends 2^31-4096..2^31-1 and the last
//                               multiples of d below 2^31 and their neighbours
//   2^22 pseudo-random (divisor < 2^31, dividend < 2^31) pairs
//
// Prints "ok <checks>" and exits 0, or the first failure and exits 1.
#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <thread>
#include <vector>

#include "../../convolution_nhwc_amd/csrc/fastdiv.h"

using cnhwc::FastDiv;
using cnhwc::fdiv;
using cnhwc::make_fastdiv;

static std::atomic<int> g_bad{0};
static std::atomic<uint64_t> g_checks{0};

static bool check(uint32_t q, uint32_t d, FastDiv f) {
    const uint32_t got = uint32_t(fdiv(int(q), f));
    if (got != q / d) {
        if (g_bad.fetch_add(1) == 0)
            std::printf("FAIL d=%u q=%u fdiv=%u true=%u (mul=%u shift=%u)\n", d, q, got, q / d, f.mul,
                        f.shift);
        return false;
    }
    return true;
}

static void small_dividends(uint32_t d0, uint32_t d1) {
    uint64_t n = 0;
    for (uint32_t d = d0; d < d1 && g_bad.load() == 0; ++d) {
        const FastDiv f = make_fastdiv(d);
        // quotient and remainder advanced together: no hardware divide per check
        uint32_t quot = 0, rem = 0;
        int bad = 0;
        for (uint32_t q = 0; q < (1u << 20); ++q) {
            bad |= uint32_t(fdiv(int(q), f)) != quot;
            if (++rem == d) { rem = 0; ++quot; }
        }
        if (bad)
            for (uint32_t q = 0; q < (1u << 20); ++q) check(q, d, f);
        n += 1u << 20;
        // the top of the range, where mulhi(q, m) + q is largest
        for (uint32_t q = 0x80000000u - 4096; q < 0x80000000u; ++q) check(q, d, f);
        const uint32_t last = (0x7fffffffu / d) * d;   // largest multiple of d below 2^31
        for (uint32_t k = 0; k < 4 && last >= k * d; ++k) {
            const uint32_t m = last - k * d;
            check(m, d, f);
            if (m > 0) check(m - 1, d, f);
            if (m < 0x7fffffffu) check(m + 1, d, f);
        }
        n += 4096 + 12;
    }
    g_checks += n;
}

static void random_pairs(uint64_t seed, int count) {
    uint64_t s = seed;
    for (int i = 0; i < count && g_bad.load() == 0; ++i) {
        // splitmix64
        s += 0x9e3779b97f4a7c15ull;
        uint64_t z = s;
        z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
        z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
        z ^= z >> 31;
        // divisors spread over every magnitude: a random 31-bit value shifted
        // right by a random amount (at least 1)
        uint32_t d = uint32_t(z & 0x7fffffffu) >> (z >> 59);
        if (d == 0) d = 1;
        const uint32_t q = uint32_t(z >> 33);
        check(q, d, make_fastdiv(d));
    }
    g_checks += uint64_t(count);
}

int main() {
    const unsigned nt = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    const uint32_t dmax = 70001;
    std::vector<std::thread> pool;
    std::atomic<uint32_t> next{1};
    for (unsigned t = 0; t < nt; ++t)
        pool.emplace_back([&] {
            for (;;) {
                const uint32_t d0 = next.fetch_add(256);
                if (d0 >= dmax) break;
                small_dividends(d0, std::min(d0 + 256, dmax));
            }
        });
    for (auto& th : pool) th.join();
    pool.clear();
    for (unsigned t = 0; t < nt; ++t) pool.emplace_back(random_pairs, 12345u + t, (1 << 22) / int(nt));
    for (auto& th : pool) th.join();
    if (g_bad.load()) return 1;
    std::printf("ok %llu\n", (unsigned long long)g_checks.load());
    return 0;
}
