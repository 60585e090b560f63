// Host check of the division by launch constants (FastDiv / fdiv in lit_internal.h) against
// the integer division it replaces, over divisors 1..5000, powers of two and their
// neighbours up to 2^24, and dividends at both ends of [0, 2^31) and around multiples of
// the divisor.  Prints "fastdiv ok" and exits 0, else the first mismatch and exits 1.
#include <cstdio>
#include <cstdint>
#include <vector>

#include "../../lightning_indexer_top_amd/csrc/lit_internal.h"

static int check(uint32_t d, int n) {
    const int want = (int)((uint32_t)n / d);
    const int got = lit::fdiv(n, lit::fast_div(d));
    if (got != want) {
        std::printf("mismatch: %d / %u = %d, fdiv gives %d\n", n, d, want, got);
        return 1;
    }
    return 0;
}

int main() {
    std::vector<uint32_t> ds;
    for (uint32_t d = 1; d <= 5000; ++d) ds.push_back(d);
    for (int e = 13; e <= 24; ++e)
        for (int k = -3; k <= 3; ++k) ds.push_back((1u << e) + (uint32_t)k);
    const int top = 0x7fffffff;
    uint64_t x = 0x9e3779b97f4a7c15ull;  // a fixed pseudo-random sequence (xorshift)
    for (uint32_t d : ds) {
        for (int n = 0; n < 3000; ++n)
            if (check(d, n)) return 1;
        for (int n = top; n > top - 3000; --n)
            if (check(d, n)) return 1;
        for (int j = 1; j <= 64; ++j) {
            const int64_t base = (int64_t)top / d / 64 * j * d;  // multiples of d across the range
            for (int k = -2; k <= 2; ++k) {
                const int64_t n = base + k;
                if (n >= 0 && n <= top && check(d, (int)n)) return 1;
            }
        }
        for (int j = 0; j < 2000; ++j) {
            x ^= x << 13, x ^= x >> 7, x ^= x << 17;
            if (check(d, (int)(x & 0x7fffffffu))) return 1;
        }
    }
    std::printf("fastdiv ok\n");
    return 0;
}
