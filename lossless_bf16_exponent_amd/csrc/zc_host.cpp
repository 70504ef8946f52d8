// Host-side parts of the C ABI: the exponent table from sigma alone or from a
// histogram, the output capacity, the header parser and the status names.
// Plain C++ with no HIP, so that the host sanitizer tests build it with g++.
//
// The table from sigma.
// The ZipCCL explainer pages ("ZipCCL: Efficient Lossless Data Compression of
// Communication Collectives for Accelerating LLM Training", section 2.A)
// replace the online histogram/sort that would find the frequent exponents by
// a bound derived from the standard deviation of a near-Gaussian tensor, so the
// remapping table is precomputed and the coder needs no online statistics.
//
// Reading used here: for X ~ N(0, sigma^2) the BF16 exponent field of X is e
// when 2^(e-127) <= |X| < 2^(e-126) (e = 1..254); e = 0 collects zero and the
// subnormals (|X| < 2^-126); e = 255 (Inf/NaN) never occurs.  With the
// half-normal tail Q(a) = P(|X| >= a) = erfc(a / (sigma sqrt 2)), the field
// probability is Q(2^(e-127)) - Q(2^(e-126)).  The seven most probable fields
// (ties to the smaller field) form the table, reported in ascending order.
//
// zc_plan_from_histogram is the online route the pages avoid: the seven
// largest counts of a measured exponent histogram, with the same tie rule and
// order.
#include <algorithm>
#include <cmath>
#include <cstring>

#include "zc.h"
#include "zc_format.h"
#include "zc_host.h"

using namespace zc;

extern "C" zc_status zc_plan_from_sigma(double sigma, zc_plan *out) {
    if (!out || !std::isfinite(sigma) || !(sigma > 0.0)) return ZC_ERR_INVALID_ARG;
    const double scale = 1.0 / (sigma * std::sqrt(2.0));

    // tail[e] = Q(2^(e-127)), e = 1..255 (tail[255] is the mass above 2^128)
    double tail[256];
    for (int e = 1; e <= 255; ++e) tail[e] = std::erfc(std::ldexp(scale, e - 127));

    double prob[256];
    prob[0] = std::erf(std::ldexp(scale, -126));
    for (int e = 1; e <= 254; ++e) prob[e] = tail[e] - tail[e + 1];
    prob[255] = 0.0;

    int order[256];
    for (int e = 0; e < 256; ++e) order[e] = e;
    std::stable_sort(order, order + 256, [&](int a, int b) { return prob[a] > prob[b]; });
    std::sort(order, order + 7);
    for (int k = 0; k < 7; ++k) out->exps[k] = static_cast<uint8_t>(order[k]);
    out->flags = 0;
    return ZC_OK;
}

extern "C" zc_status zc_plan_from_histogram(const uint64_t *hist, zc_plan *out) {
    if (!hist || !out) return ZC_ERR_INVALID_ARG;
    int order[256];
    for (int e = 0; e < 256; ++e) order[e] = e;
    std::stable_sort(order, order + 256, [&](int a, int b) { return hist[a] > hist[b]; });
    std::sort(order, order + 7);
    for (int k = 0; k < 7; ++k) out->exps[k] = static_cast<uint8_t>(order[k]);
    out->flags = 0;
    return ZC_OK;
}

bool zc_plan_is_valid(const zc_plan *p) {
    if (!p || (p->flags & ~(uint8_t)ZC_PLAN_RAW_FALLBACK)) return false;
    for (int k = 1; k < 7; ++k)
        if (p->exps[k] <= p->exps[k - 1]) return false;
    return true;
}

extern "C" uint64_t zc_max_compressed_bytes(uint64_t n) {
    if (n > kMaxElems) return 0;
    return layout_for(n).off_scratch;  // the largest stream, coded or raw, rounded up to 128
}

extern "C" uint64_t zc_compress_workspace_bytes(uint64_t n) {
    if (n > kMaxElems) return 0;
    return (scratch_for(n).bytes + 255u) & ~uint64_t(255u);
}

static uint32_t rd32(const uint8_t *p) {
    uint32_t v;
    std::memcpy(&v, p, 4);
    return v;
}
static uint64_t rd64(const uint8_t *p) {
    uint64_t v;
    std::memcpy(&v, p, 8);
    return v;
}

extern "C" zc_status zc_read_header(const void *host_header, uint64_t len, zc_stream_info *out) {
    if (!host_header || !out) return ZC_ERR_INVALID_ARG;
    if (len < kHeaderBytes) return ZC_ERR_CORRUPT;
    const uint8_t *h = static_cast<const uint8_t *>(host_header);
    const uint64_t n = rd64(h + 8);
    if (rd32(h) != kMagic || rd32(h + 4) != ((uint32_t)kVersion | (kHeaderBytes << 16)) || n > kMaxElems ||
        rd32(h + 16) != kGroup)
        return ZC_ERR_CORRUPT;
    const Layout L = layout_for(n);
    zc_plan p;
    std::memcpy(p.exps, h + 24, 7);
    p.flags = 0;
    const uint32_t mode = h[31];
    const uint64_t E = rd64(h + 32), total = rd64(h + 40);
    if (mode != kModeCoded && mode != kModeRaw) return ZC_ERR_CORRUPT;
    const uint64_t expect = mode == kModeRaw ? kHeaderBytes + 2 * n : L.off_zp + E;
    if (rd32(h + 20) != L.groups || !zc_plan_is_valid(&p) || E > n || total != expect) return ZC_ERR_CORRUPT;
    for (int i = 48; i < 128; ++i)
        if (h[i]) return ZC_ERR_CORRUPT;
    out->n = n;
    out->zero_points = E;
    out->total_bytes = total;
    out->groups = (uint32_t)L.groups;
    out->plan = p;
    out->raw = mode == kModeRaw ? 1u : 0u;
    return ZC_OK;
}

extern "C" const char *zc_status_string(zc_status s) {
    switch (s) {
        case ZC_OK: return "ok";
        case ZC_ERR_INVALID_ARG: return "invalid argument";
        case ZC_ERR_CAPACITY: return "output or workspace capacity below what the call needs";
        case ZC_ERR_MISALIGNED: return "misaligned buffer";
        case ZC_ERR_CORRUPT: return "corrupt stream";
        case ZC_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}
