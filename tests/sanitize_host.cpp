// Host program of the sanitizer test: exercises every host planner call of
// libzero_mi355x (zero_host.cpp) and the oracle's C functions over small grids,
// error paths included, in a build with AddressSanitizer and UBSan.  Exits
// non-zero on the first wrong result; the sanitizers abort on any report.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "zero.h"

extern "C" {
int orc_partition(uint64_t psi, uint32_t nd, uint32_t rank, uint64_t *begin, uint64_t *end);
int orc_mem_bytes(uint32_t stage, uint64_t psi, uint32_t nd, uint32_t k, uint64_t *bytes);
void orc_grad_stats(const uint16_t *g, int is_bf16, uint64_t n, double inv_scale,
                    double *sq_norm, uint32_t *overflow);
}

#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            return 1;                                                   \
        }                                                               \
    } while (0)

int main()
{
    // partition: agrees with the oracle and tiles [0, psi) for small grids
    for (uint64_t psi = 0; psi <= 300; ++psi)
        for (uint32_t nd = 1; nd <= 33; ++nd) {
            uint64_t prev = 0;
            for (uint32_t r = 0; r < nd; ++r) {
                uint64_t b, e, ob, oe;
                CHECK(zero_partition(psi, nd, r, &b, &e) == ZERO_OK);
                CHECK(orc_partition(psi, nd, r, &ob, &oe) == 0);
                CHECK(b == ob && e == oe && b == prev && e >= b);
                prev = e;
            }
            CHECK(prev == psi);
        }
    uint64_t b, e;
    CHECK(zero_partition(10, 0, 0, &b, &e) == ZERO_EINVAL);
    CHECK(zero_partition(10, 3, 3, &b, &e) == ZERO_EINVAL);
    CHECK(zero_partition(10, 3, 0, nullptr, &e) == ZERO_EINVAL);
    CHECK(std::strlen(zero_last_error()) > 0);
    for (int s = 0; s <= 5; ++s)
        CHECK(zero_status_str((zero_status)s) != nullptr);

    // accounting: agrees with the oracle; overflow is an error, not a wrap
    for (uint32_t stage = 0; stage <= 3; ++stage)
        for (uint64_t psi : {0ull, 1ull, 7500000000ull, 1557611200ull})
            for (uint32_t nd : {1u, 7u, 64u, 1024u}) {
                uint64_t x, ox;
                CHECK(zero_mem_bytes(stage, psi, nd, 12, &x) == ZERO_OK);
                CHECK(orc_mem_bytes(stage, psi, nd, 12, &ox) == 0 && x == ox);
            }
    uint64_t x;
    CHECK(zero_mem_bytes(4, 1, 1, 12, &x) == ZERO_EINVAL);
    CHECK(zero_mem_bytes(0, UINT64_MAX / 2, 1, 12, &x) == ZERO_EINVAL);

    // bucket plan over random ragged lists (zero-size tensors included)
    std::mt19937_64 rng(1);
    for (int trial = 0; trial < 300; ++trial) {
        const uint32_t nt = 1 + rng() % 12;
        std::vector<uint64_t> numel(nt);
        uint64_t psi = 0;
        for (auto &k : numel) {
            k = rng() % 4 == 0 ? 0 : rng() % 1000;
            psi += k;
        }
        const uint64_t B = 1 + rng() % 700;
        const uint64_t lo = psi ? rng() % (psi + 1) : 0, hi = lo + (psi - lo ? rng() % (psi - lo + 1) : 0);
        uint64_t count = 0;
        CHECK(zero_bucket_plan(numel.data(), nt, B, lo, hi, nullptr, 0, &count) ==
              (count ? ZERO_ENOSPC : ZERO_OK) || count == 0);
        std::vector<zero_segment> segs(count + 1);
        uint64_t n2 = 0;
        CHECK(zero_bucket_plan(numel.data(), nt, B, lo, hi, segs.data(), count, &n2) == ZERO_OK);
        CHECK(n2 == count);
        uint64_t covered = 0;
        for (uint64_t i = 0; i < count; ++i) {
            const auto &sg = segs[i];
            CHECK(sg.dst_off == covered && sg.len > 0 && sg.tensor < nt);
            CHECK(sg.src_off + sg.len <= numel[sg.tensor]);
            covered += sg.len;
        }
        CHECK(covered == hi - lo);
        if (count > 1) {
            uint64_t n3 = 0;
            CHECK(zero_bucket_plan(numel.data(), nt, B, lo, hi, segs.data(), count - 1, &n3) ==
                  ZERO_ENOSPC);
            CHECK(n3 == count);
        }
    }
    uint64_t nseg;
    const uint64_t one = 5;
    CHECK(zero_bucket_plan(&one, 1, 0, 0, 5, nullptr, 0, &nseg) == ZERO_EINVAL);
    CHECK(zero_bucket_plan(&one, 1, 2, 3, 2, nullptr, 0, &nseg) == ZERO_EINVAL);
    CHECK(zero_bucket_plan(&one, 1, 2, 0, 6, nullptr, 0, &nseg) == ZERO_EINVAL);

    // state layout
    uint64_t offs[5];
    CHECK(zero_state_layout(1557611200ull, 200ull << 30, offs) == ZERO_OK);
    for (int i = 1; i < 5; ++i)
        CHECK(offs[i] - offs[i - 1] == offs[1] && offs[1] % (2u << 20) == 0);
    CHECK(zero_state_layout(1u << 20, 18u << 20, offs) == ZERO_ENOSPC);
    CHECK(zero_state_layout(1u << 20, 1ull << 30, nullptr) == ZERO_EINVAL);

    // the oracle's statistics over every fp16 pattern (reads stay in bounds)
    std::vector<uint16_t> g(1 << 16);
    for (uint32_t i = 0; i < g.size(); ++i)
        g[i] = (uint16_t)i;
    double sq;
    uint32_t ov;
    orc_grad_stats(g.data(), 0, g.size(), 1.0, &sq, &ov);
    CHECK(ov == 1);
    orc_grad_stats(g.data(), 0, 0x7c00, 1.0, &sq, &ov);  // the finite positive ones
    CHECK(ov == 0 && std::isfinite(sq) && sq > 0);
    std::puts("sanitized host checks passed");
    return 0;
}
