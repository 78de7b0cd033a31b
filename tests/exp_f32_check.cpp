// Host build of the correctly rounded fp32 exponential (exp_f32_rn.h), checked
// against the C library: for every fp32 x in [lo_bits, hi_bits) with stride `step`,
// compares exp_f32_rn(x) with (float)expl(x) (x87 extended precision, so a
// wrong fp32 rounding there needs exp(x) within 2^-63 of a rounding midpoint)
// and counts the x where (float)exp((double)x) (one rounding from a double
// exponential) differs.  Prints: checked, mismatches vs expl, differences vs
// exp, then up to 20 mismatching inputs as hex bit patterns.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "exp_f32_rn.h"

static float from_bits(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }

int main(int argc, char** argv) {
    const uint64_t step = argc > 1 ? strtoull(argv[1], nullptr, 0) : 1;
    const int nt = argc > 2 ? atoi(argv[2]) : 8;
    struct Res { uint64_t n = 0, bad = 0, diff_exp = 0; std::vector<uint32_t> ex; };
    std::vector<Res> res(nt);
    std::vector<std::thread> th;
    for (int t = 0; t < nt; ++t)
        th.emplace_back([&, t] {
            Res& r = res[t];
            for (uint64_t u = (uint64_t)t * step; u < (1ull << 32); u += (uint64_t)nt * step) {
                const float x = from_bits((uint32_t)u);
                const float got = w8a8_test::exp_f32_rn(x);
                const float want = (float)expl((long double)x);
                ++r.n;
                const bool same = (got == want && std::signbit(got) == std::signbit(want)) ||
                                  (std::isnan(got) && std::isnan(want));
                if (!same) {
                    ++r.bad;
                    if (r.ex.size() < 20) r.ex.push_back((uint32_t)u);
                }
                const float viad = (float)std::exp((double)x);
                if (!(viad == want || (std::isnan(viad) && std::isnan(want)))) ++r.diff_exp;
            }
        });
    for (auto& x : th) x.join();
    uint64_t n = 0, bad = 0, de = 0;
    std::vector<uint32_t> ex;
    for (auto& r : res) {
        n += r.n; bad += r.bad; de += r.diff_exp;
        for (auto e : r.ex) if (ex.size() < 20) ex.push_back(e);
    }
    printf("%llu %llu %llu\n", (unsigned long long)n, (unsigned long long)bad, (unsigned long long)de);
    for (auto e : ex) printf("%08x\n", e);
    return 0;
}
