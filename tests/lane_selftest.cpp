// Host build of the codec's per-lane bit helpers, checked bit for bit against
// per-element definitions written out here (split into sign/exponent/mantissa,
// code = position in a window of seven exponents, plane b = bit b of the code).
// Built by tests/test_host.py with the same compiler as the library; no GPU.
#include <cstdio>
#include <cstdlib>

#include "zc_lane.h"

using namespace zc;

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd() {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 16);
}

static int failures = 0;
#define CHECK(cond)                                                         \
    do {                                                                    \
        if (!(cond)) {                                                      \
            if (failures++ < 10) std::printf("FAIL line %d: %s\n", __LINE__, #cond); \
        }                                                                   \
    } while (0)

int main() {
    for (int iter = 0; iter < 200000; ++iter) {
        uint32_t d[4];
        for (auto &w : d) w = rnd();
        uint16_t x[8];
        for (int i = 0; i < 8; ++i) x[i] = (uint16_t)(d[i / 2] >> (16 * (i % 2)));
        // sign+mantissa and exponent bytes
        uint32_t sm_lo = sign_mantissa4(d[0], d[1]), sm_hi = sign_mantissa4(d[2], d[3]);
        uint32_t t[4];
        for (int i = 0; i < 4; ++i) t[i] = exponent_high(d[i]);
        uint32_t e_lo = exponents4(t[0], t[1]), e_hi = exponents4(t[2], t[3]);
        for (int i = 0; i < 8; ++i) {
            uint32_t sm = get_byte8(sm_lo, sm_hi, i), e = get_byte8(e_lo, e_hi, i);
            CHECK(sm == (((x[i] >> 15) << 7) | (x[i] & 0x7Fu)));
            CHECK(e == ((x[i] >> 7) & 0xFFu));
        }
        // window codes for a window starting at first = 1..249
        uint32_t first = 1 + rnd() % 249, base = first - 1;
        uint32_t base_hi = (base << 8) | (base << 24);
        uint32_t c_lo = window_codes4(t[0], t[1], base_hi), c_hi = window_codes4(t[2], t[3], base_hi);
        uint32_t code[8];
        for (int i = 0; i < 8; ++i) {
            uint32_t e = (x[i] >> 7) & 0xFFu;
            code[i] = (e >= first && e < first + 7) ? e - first + 1 : 0;
            CHECK((get_byte8(c_lo, c_hi, i) & 7u) == code[i]);
            CHECK(get_byte8(c_lo, c_hi, i) <= 8u);
        }
        // planes: byte b holds bit b of the codes, value k in bit k
        uint32_t planes = codes_to_planes(c_lo, c_hi) & 0x00FFFFFFu;
        uint32_t zmask = 0;
        for (int b = 0; b < 3; ++b)
            for (int k = 0; k < 8; ++k) CHECK(((planes >> (8 * b + k)) & 1u) == ((code[k] >> b) & 1u));
        for (int k = 0; k < 8; ++k) zmask |= (code[k] == 0u) << k;
        CHECK(zero_point_mask(planes) == zmask);
        // inverse transpose
        uint32_t r_lo, r_hi;
        planes_to_codes(planes, r_lo, r_hi);
        for (int k = 0; k < 8; ++k) CHECK(get_byte8(r_lo, r_hi, k) == code[k]);
        // arbitrary plane bytes decode to the bits they hold
        uint32_t p2 = rnd() & 0x00FFFFFFu;
        planes_to_codes(p2, r_lo, r_hi);
        for (int k = 0; k < 8; ++k) {
            uint32_t c = ((p2 >> k) & 1u) | (((p2 >> (8 + k)) & 1u) << 1) | (((p2 >> (16 + k)) & 1u) << 2);
            CHECK(get_byte8(r_lo, r_hi, k) == c);
        }
        // table lookup through perm: code byte -> exponent byte
        uint32_t tbl_lo = rnd() & 0xFFFFFF00u, tbl_hi = rnd();
        uint32_t q_lo = perm(tbl_hi, tbl_lo, r_lo), q_hi = perm(tbl_hi, tbl_lo, r_hi);
        for (int k = 0; k < 8; ++k) {
            uint32_t c = get_byte8(r_lo, r_hi, k);
            CHECK(get_byte8(q_lo, q_hi, k) == get_byte8(tbl_lo, tbl_hi, c));
        }
        // rebuild inverts the split
        uint32_t o0, o1, o2, o3;
        rebuild4(sm_lo, e_lo, o0, o1);
        rebuild4(sm_hi, e_hi, o2, o3);
        CHECK(o0 == d[0] && o1 == d[1] && o2 == d[2] && o3 == d[3]);
        // get byte: the little-endian byte order of the 8-byte value
        uint32_t lo = rnd(), hi = rnd();
        const uint64_t v = ((uint64_t)hi << 32) | lo;
        for (uint32_t j = 0; j < 8; ++j) CHECK(get_byte8(lo, hi, j) == ((v >> (8 * j)) & 0xFFu));
    }
    if (failures) {
        std::printf("%d failures\n", failures);
        return 1;
    }
    std::printf("lane helpers: all checks passed\n");
    return 0;
}
