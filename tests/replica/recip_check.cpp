// Check of the host reciprocals the tree-attention kernels divide by
// (attn_plan.hpp: recip_of, div_by): floor(n / d) for 0 <= n < 2^31 against the
// plain division, for every divisor up to 4096 on edge and random dividends,
// random divisors up to 2^31 - 1 on the dividends around their multiples, and a
// few divisors over every dividend.  Prints "ok".
#define EAGLE_HD
#include "../../draft_tree_verification_eagle_amd/csrc/attn_plan.hpp"

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>

using namespace eagle::plan;

static void fail(uint32_t n, uint32_t d) {
    std::fprintf(stderr, "wrong quotient: n=%u d=%u\n", n, d);
    std::exit(1);
}
static void one(uint32_t n, uint32_t d, const Recip& r) {
    if (n >= (1u << 31)) return;
    if (div_by(n, r) != n / d) fail(n, d);
}
static void around_multiples(uint32_t d, const Recip& r, std::mt19937_64& g) {
    const uint32_t top = (1u << 31) - 1;
    for (int k = 0; k < 64; ++k) {
        const uint64_t q = k < 32 ? (uint64_t)k : g() % ((uint64_t)top / d + 1);
        const uint64_t base = q * d;
        for (int e = -2; e <= 2; ++e) {
            const int64_t n = (int64_t)base + e;
            if (n >= 0 && n <= top) one((uint32_t)n, d, r);
        }
    }
    for (int e = 0; e < 4; ++e) one(top - e, d, r);
}

int main() {
    std::mt19937_64 g(7);
    for (uint32_t d = 1; d <= 4096; ++d) {
        const Recip r = recip_of(d);
        for (uint32_t n = 0; n < 4096; ++n) one(n, d, r);
        around_multiples(d, r, g);
        for (int k = 0; k < 256; ++k) one((uint32_t)(g() & 0x7fffffffu), d, r);
    }
    for (int k = 0; k < 20000; ++k) {
        const uint32_t d = 1 + (uint32_t)(g() % 0x7ffffffeu);
        const Recip r = recip_of(d);
        around_multiples(d, r, g);
        for (int j = 0; j < 16; ++j) one((uint32_t)(g() & 0x7fffffffu), d, r);
    }
    for (int shift = 0; shift < 31; ++shift) {  // powers of two and their neighbours
        for (int e = -1; e <= 1; ++e) {
            const int64_t d = ((int64_t)1 << shift) + e;
            if (d < 1 || d > 0x7fffffff) continue;
            const Recip r = recip_of((uint32_t)d);
            around_multiples((uint32_t)d, r, g);
        }
    }
    const uint32_t full[] = {61, 0x7fffffffu};
    for (uint32_t d : full) {
        const Recip r = recip_of(d);
        for (uint32_t n = 0; n < (1u << 31); ++n)
            if ((uint32_t)((n * r.m) >> r.sh) != n / d) fail(n, d);
    }
    std::printf("ok\n");
    return 0;
}
