// Host-side exponent table from sigma alone.
//
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

#include "zc.h"

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
