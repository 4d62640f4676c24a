// Host check of the per-head row addressing in kernels.h: the multiply-shift
// quotient must equal r / heads for every divisor the library accepts and
// for row indices across the whole supported range (R < 2^30), including
// the values next to each multiple of heads and the top of the range.
// Prints the number of failures and exits non-zero on any.
#include <cstdio>
#include <cstdint>
#include <random>
#include <vector>

#include "kernels.h"

static uint32_t quotient(uint32_t n, const rmsn::RowMap& m)
{
    // the device computes the high half with __umulhi; the same on the host
    const uint32_t hi = (uint32_t)(((uint64_t)n * m.magic) >> 32);
    return (hi + ((n - hi) >> 1)) >> (m.shift - 1);
}

int main()
{
    std::mt19937_64 rng(12345);
    long fails = 0, checks = 0;
    auto check = [&](uint32_t n, uint32_t d, const rmsn::RowMap& m) {
        ++checks;
        if (quotient(n, m) != n / d) {
            if (fails < 10) std::printf("heads=%u r=%u: got %u want %u\n", d, n, quotient(n, m), n / d);
            ++fails;
        }
    };
    std::vector<uint32_t> divisors;
    for (uint32_t d = 2; d <= 4096; ++d) divisors.push_back(d);
    for (int i = 0; i < 2000; ++i) divisors.push_back(2 + (uint32_t)(rng() % ((1u << 30) - 2)));
    const uint32_t top = (1u << 30) - 1;
    for (uint32_t d : divisors) {
        const rmsn::RowMap m = rmsn::make_row_map(d, 0, 0);
        for (uint32_t n = 0; n < 3 * d && n < 20000; ++n) check(n, d, m);
        for (uint32_t q = top / d - 3; q <= top / d; ++q)
            for (int e = -1; e <= 1; ++e) {
                const int64_t n = (int64_t)q * d + e;
                if (n >= 0 && n <= top) check((uint32_t)n, d, m);
            }
        for (int i = 0; i < 2000; ++i) check((uint32_t)(rng() % (top + 1ull)), d, m);
        for (uint32_t n = 0xFFFFFFFFu - 4; n != 0; ++n) check(n, d, m);  // beyond the range, still exact
    }
    std::printf("%ld checks, %ld failures\n", checks, fails);
    return fails != 0;
}
