// Host-side check of the single-read LayerNorm kernel's exchange tags
// (normalization_ln_forward_amd/csrc/ln_tag.hpp, the same functions the
// kernel calls): for every generation the tag is in [1, 255], differs from
// the previous generation's, and accepts none of the words other writers
// leave in the exchange slots: zero (the zeroing kernel) and element counts
// (the split and last-workgroup-merges schedules store an integer n in the
// first word).  A tagged word carries its tag and untags to the value with
// its low 8 mantissa bits cleared.  Runs on the CPU only.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "ln_tag.hpp"

using namespace normfwd;

static int fails = 0;
#define CHECK(c, ...)                        \
    do {                                     \
        if (!(c)) {                          \
            if (fails < 20) {                \
                std::printf("FAIL: ");       \
                std::printf(__VA_ARGS__);    \
                std::printf("\n");           \
            }                                \
            ++fails;                         \
        }                                    \
    } while (0)

int main()
{
    // every generation a workspace can hold, plus out-of-range words (a
    // workspace that was never zeroed) that the kernel also reduces mod 255
    const uint32_t extra[] = {255u, 256u, 511u, 65535u, 0x7FFFFFFFu, 0xFFFFFFFEu, 0xFFFFFFFFu};
    for (int pass = 0; pass < 2; ++pass) {
        const int count = pass == 0 ? 255 : (int)(sizeof(extra) / sizeof(extra[0]));
        for (int i = 0; i < count; ++i) {
            const uint32_t g = pass == 0 ? (uint32_t)i : extra[i];
            const uint32_t next = ln_next_generation(g);
            CHECK(next < 255u, "generation %u -> %u out of range", g, next);
            const uint32_t tag = ln_tag_of(next);
            CHECK(tag >= 1u && tag <= 255u, "tag %u of generation %u", tag, next);
            if (g < 255u) CHECK(tag != ln_tag_of(g), "generations %u and %u share tag %u", g, next, tag);
            CHECK(!ln_has_tag(0.0, tag), "zero accepted under tag %u", tag);
            CHECK(!ln_has_tag(-0.0, tag), "-0 accepted under tag %u", tag);
            // element counts: every integer up to 2^20, then sparse up to 2^44
            for (int64_t n = 1; n <= (1 << 20); ++n)
                if (ln_has_tag((double)n, tag)) {
                    CHECK(false, "count %lld accepted under tag %u", (long long)n, tag);
                    break;
                }
            for (int64_t n = (1 << 20); n < ((int64_t)1 << 44); n = n * 3 + 7)
                CHECK(!ln_has_tag((double)n, tag), "count %lld accepted under tag %u", (long long)n, tag);
            // round trip on values of every magnitude and sign
            const double vals[] = {1.0, -1.0, 100.000123456789, 1e-300, -3.5e17, 0.1, 419.4304, 6.02e23};
            for (double v : vals) {
                const double w = ln_tag_word(v, tag);
                CHECK(ln_has_tag(w, tag), "tagged %g lacks tag %u", v, tag);
                CHECK(ln_untag(w) == ln_untag(v), "untag(tag(%g)) changed the value", v);
                CHECK(std::fabs(ln_untag(w) - v) <= std::ldexp(std::fabs(v), -44), "tag moved %g too far", v);
                CHECK(!ln_has_tag(w, ln_tag_of(ln_next_generation(next))), "tagged %g accepted by the next generation", v);
            }
        }
    }
    if (fails) {
        std::printf("ln_tag_test: %d failures\n", fails);
        return 1;
    }
    std::printf("ln_tag_test: ok\n");
    return 0;
}
