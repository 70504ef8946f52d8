// Host check of the library's host-side C ABI (zc_host.cpp) and of the layout
// arithmetic it shares with the kernels (zc_format.h), built with
// -fsanitize=address,undefined by tests/test_host.py: every call on edge and
// random inputs must stay in bounds and free of undefined behaviour, and
// return what the header documents.  No GPU; no oracle (the oracle's own
// sanitizer run is separate).
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

#include "zc.h"
#include "zc_format.h"

using namespace zc;

static int failures = 0;
#define CHECK(cond)                                                                      \
    do {                                                                                 \
        if (!(cond)) {                                                                   \
            if (failures++ < 10) std::printf("FAIL line %d: %s\n", __LINE__, #cond);     \
        }                                                                                \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t rnd() {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return rng_state;
}

static bool ascending(const zc_plan &p) {
    for (int k = 1; k < 7; ++k)
        if (p.exps[k] <= p.exps[k - 1]) return false;
    return p.flags == 0;
}

static void put32(uint8_t *h, int off, uint32_t v) { std::memcpy(h + off, &v, 4); }
static void put64(uint8_t *h, int off, uint64_t v) { std::memcpy(h + off, &v, 8); }

// A header as the encoder writes it (coded or raw form).
static void make_header(uint8_t *h, uint64_t n, const uint8_t *exps, uint64_t E, bool raw) {
    std::memset(h, 0, 128);
    const Layout L = layout_for(n);
    put32(h, 0, kMagic);
    put32(h, 4, (uint32_t)kVersion | (kHeaderBytes << 16));
    put64(h, 8, n);
    put32(h, 16, kGroup);
    put32(h, 20, (uint32_t)L.groups);
    std::memcpy(h + 24, exps, 7);
    h[31] = raw ? 1 : 0;
    put64(h, 32, E);
    put64(h, 40, raw ? kHeaderBytes + 2 * n : L.off_zp + E);
}

int main() {
    // ---- the table from sigma: finite positive sigma over the whole double range
    const double special[] = {0.0, -1.0, std::numeric_limits<double>::infinity(),
                              -std::numeric_limits<double>::infinity(), std::nan("")};
    for (double s : special) {
        zc_plan p;
        CHECK(zc_plan_from_sigma(s, &p) == ZC_ERR_INVALID_ARG);
    }
    CHECK(zc_plan_from_sigma(1.0, nullptr) == ZC_ERR_INVALID_ARG);
    for (double l2 = -1074.0; l2 < 1024.0; l2 += 0.37) {
        zc_plan p;
        const double s = std::ldexp(1.0, (int)std::floor(l2)) * std::exp2(l2 - std::floor(l2));
        if (!(s > 0.0) || !std::isfinite(s)) continue;
        CHECK(zc_plan_from_sigma(s, &p) == ZC_OK);
        CHECK(ascending(p));
    }
    {
        zc_plan p;
        CHECK(zc_plan_from_sigma(std::numeric_limits<double>::denorm_min(), &p) == ZC_OK && ascending(p));
        CHECK(zc_plan_from_sigma(std::numeric_limits<double>::max(), &p) == ZC_OK && ascending(p));
        CHECK(zc_plan_from_sigma(0.02, &p) == ZC_OK && p.exps[0] == 116 && p.exps[6] == 122);
    }

    // ---- the table from a histogram: all-zero, single-bin, random, extreme counts
    {
        uint64_t h[256];
        zc_plan p;
        CHECK(zc_plan_from_histogram(nullptr, &p) == ZC_ERR_INVALID_ARG);
        CHECK(zc_plan_from_histogram(h, nullptr) == ZC_ERR_INVALID_ARG);
        std::memset(h, 0, sizeof(h));
        CHECK(zc_plan_from_histogram(h, &p) == ZC_OK && ascending(p) && p.exps[0] == 0 && p.exps[6] == 6);
        h[255] = ~0ull;
        CHECK(zc_plan_from_histogram(h, &p) == ZC_OK && ascending(p) && p.exps[6] == 255);
        for (int it = 0; it < 2000; ++it) {
            for (auto &v : h) v = (rnd() & 3) ? rnd() >> (rnd() & 63) : 0;
            CHECK(zc_plan_from_histogram(h, &p) == ZC_OK && ascending(p));
        }
    }

    // ---- capacity and layout arithmetic over edge and random sizes
    std::vector<uint64_t> sizes = {0, 1, 63, 64, 65, 4095, 4096, 4097, 8191, 8192, 8193, 1u << 20,
                                   kMaxElems - 1, kMaxElems};
    for (int it = 0; it < 20000; ++it) sizes.push_back(rnd() % (kMaxElems + 1));
    for (uint64_t n : sizes) {
        const Layout L = layout_for(n);
        const Scratch S = scratch_for(n);
        const uint64_t cap = zc_max_compressed_bytes(n);
        CHECK(L.off_p0 % 128 == 0 && L.off_p1 % 128 == 0 && L.off_p2 % 128 == 0 && L.off_tab % 128 == 0 &&
              L.off_zp % 128 == 0 && L.off_scratch % 128 == 0);
        CHECK(L.off_p0 >= kHeaderBytes + n && L.off_tab >= L.off_p2 + 8 * ((n + 63) / 64));
        CHECK(L.off_zp >= L.off_tab + 4 * (L.groups + 1));
        CHECK(L.off_scratch >= L.off_zp + n);                      // the largest stream fits before the scratch
        CHECK(L.off_scratch >= kHeaderBytes + 2 * n);              // so does the raw form
        CHECK(S.staging >= S.group_words && S.bytes == S.staging + enc_blocks(n) * (uint64_t)kEncSpan);
        CHECK(cap == L.off_scratch);                               // the stream bound
        const uint64_t ws = zc_compress_workspace_bytes(n);
        CHECK(ws % 256 == 0 && ws >= S.bytes && ws < S.bytes + 256);
        CHECK(S.decision % kWordBytes == 0 && S.status % kWordBytes == 0 && S.span_words >= S.status + kWordBytes);
        // every region in order, none overlapping the next: the 8-byte epoch
        // between the status word and the span words, each word array sized
        // for its units
        const uint64_t nb = enc_blocks(n), nr = ceil_div(nb, kRun), nc = ceil_div(nr, kChunkRuns);
        const uint64_t ng = ceil_div(nb, kGroupSpans);
        CHECK(S.status >= S.decision + kWordBytes && S.epoch >= S.status + kWordBytes && S.epoch % 8 == 0);
        CHECK(S.span_words >= S.epoch + 8 && S.run_words >= S.span_words + kWordBytes * nb);
        CHECK(S.chunk_words >= S.run_words + kWordBytes * nr && S.group_words >= S.chunk_words + kWordBytes * nc);
        CHECK(S.staging >= S.group_words + kWordBytes * ng);
        CHECK(S.span_words % 128 == 0 && S.staging % 128 == 0);
    }
    CHECK(zc_max_compressed_bytes(kMaxElems + 1) == 0);
    CHECK(zc_max_compressed_bytes(~0ull) == 0);
    CHECK(zc_compress_workspace_bytes(kMaxElems + 1) == 0);

    // ---- the header parser: valid headers, every single-byte corruption, random bytes, short lengths
    {
        uint8_t h[128];
        const uint8_t exps[7] = {116, 117, 118, 119, 120, 121, 122};
        zc_stream_info info;
        CHECK(zc_read_header(nullptr, 128, &info) == ZC_ERR_INVALID_ARG);
        make_header(h, 1000, exps, 10, false);
        CHECK(zc_read_header(h, 128, nullptr) == ZC_ERR_INVALID_ARG);
        for (uint64_t len = 0; len < 128; ++len) CHECK(zc_read_header(h, len, &info) == ZC_ERR_CORRUPT);
        const uint64_t ns[] = {0, 1, 4096, 1000003, kMaxElems};
        for (uint64_t n : ns)
            for (int raw = 0; raw < 2; ++raw) {
                const uint64_t E = n / 3;
                make_header(h, n, exps, E, raw != 0);
                CHECK(zc_read_header(h, 128, &info) == ZC_OK);
                CHECK(info.n == n && info.zero_points == E && info.raw == (uint32_t)raw);
                for (int pos = 0; pos < 128; ++pos)
                    for (int bit = 0; bit < 8; ++bit) {
                        uint8_t c[128];
                        std::memcpy(c, h, 128);
                        c[pos] ^= (uint8_t)(1u << bit);
                        const zc_status st = zc_read_header(c, 128, &info);
                        CHECK(st == ZC_OK || st == ZC_ERR_CORRUPT);
                    }
            }
        for (int it = 0; it < 100000; ++it) {
            for (auto &b : h) b = (uint8_t)rnd();
            if (it & 1) put32(h, 0, kMagic);
            if (it & 2) put32(h, 4, (uint32_t)kVersion | (kHeaderBytes << 16));
            if (it & 4) put32(h, 16, kGroup);
            const zc_status st = zc_read_header(h, 128, &info);
            CHECK(st == ZC_OK || st == ZC_ERR_CORRUPT);
        }
    }

    // ---- status names
    for (int s = -3; s < 10; ++s) CHECK(zc_status_string((zc_status)s) != nullptr);

    if (failures) {
        std::printf("%d failures\n", failures);
        return 1;
    }
    std::printf("host ABI ok\n");
    return 0;
}
