/*
 * CPU oracle for the BF16 exponent-coding codec -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load or run this file.  The product path (the HIP library) shares no code,
 * header, table or constant with it.
 *
 * What it computes follows the explainer pages of
 *   "ZipCCL: Efficient Lossless Data Compression of Communication Collectives
 *    for Accelerating LLM Training" (gist.science, fr/ja/ko pages),
 * technical summary section 2 ("Methodology"):
 *   - section 2.A: the top-7 exponents follow from the standard deviation of a
 *     near-Gaussian tensor, so the exponent table is precomputed from sigma
 *     with no online histogram;
 *   - section 2.B: every BF16 word is split into sign+mantissa bits and the
 *     8-bit exponent; an exponent among the top 7 is remapped to a 3-bit code
 *     001..111, any other exponent gets the "zero-point" code 000 and its full
 *     8 bits go to a separate zero-point array (16 -> 11 bits when no value
 *     takes the zero-point path);
 *   - section 2.C: the 3-bit codes are kept as three separate 1-bit arrays and
 *     data blocks are padded to 128-byte boundaries;
 *   - section 2.D: a reduce-scatter may run as a zipped all-to-all followed by
 *     a local reduction (zco_decode_reduce);
 *   - the online statistics that section 2.A avoids, for comparison: the
 *     exponent histogram with its top-7 plan, and a sigma estimate
 *     (zco_exponent_histogram, zco_plan_from_histogram, zco_estimate_sigma,
 *     at the end of this file).
 * Every step is written as a plain per-element loop in the pages' order; no
 * blocking, fusion or reordering.  Where the pages are silent (which exponent
 * gets which code, bit order in the planes, the header, the table of
 * zero-point offsets) the reading used is stated at the point of use below.
 *
 * Byte layout of one compressed stream (all integers little-endian, every
 * section starts on a 128-byte boundary, every pad byte is zero):
 *   header  128 B                      magic, version, n, exps, counts
 *   SM      n B                        sign+mantissa byte per element
 *   plane0  8*ceil(n/64) B             bit 0 of every code
 *   plane1  8*ceil(n/64) B             bit 1 of every code
 *   plane2  8*ceil(n/64) B             bit 2 of every code
 *   TAB     4*(NG+1) B, NG=ceil(n/4096)  zero-point count before each group
 *   ZP      E B                        full exponent of every zero-point value
 * Header byte 31 is the mode: 0 for this coded layout, 1 for the raw fallback
 * (zco_encode_fallback): the header, then the n words unchanged.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ZCO_OK 0
#define ZCO_ERR_INVALID_ARG 1
#define ZCO_ERR_CAPACITY 2
#define ZCO_ERR_CORRUPT 4

#define ZCO_MAGIC 0x3143435Au /* bytes "ZCC1" */
#define ZCO_VERSION 1u
#define ZCO_HEADER_BYTES 128u
#define ZCO_GROUP 4096u
#define ZCO_MODE_CODED 0u /* header byte 31 */
#define ZCO_MODE_RAW 1u

/* ------------------------------------------------------------------------ */
/* little helpers                                                            */
/* ------------------------------------------------------------------------ */

static uint64_t round_up_128(uint64_t x) { return (x + 127u) / 128u * 128u; }

static void put_u16(uint8_t *p, uint16_t v) {
    p[0] = (uint8_t)(v & 0xFF);
    p[1] = (uint8_t)(v >> 8);
}
static void put_u32(uint8_t *p, uint32_t v) {
    for (int i = 0; i < 4; ++i) p[i] = (uint8_t)(v >> (8 * i));
}
static void put_u64(uint8_t *p, uint64_t v) {
    for (int i = 0; i < 8; ++i) p[i] = (uint8_t)(v >> (8 * i));
}
static uint16_t get_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t get_u32(const uint8_t *p) {
    uint32_t v = 0;
    for (int i = 3; i >= 0; --i) v = (v << 8) | p[i];
    return v;
}
static uint64_t get_u64(const uint8_t *p) {
    uint64_t v = 0;
    for (int i = 7; i >= 0; --i) v = (v << 8) | p[i];
    return v;
}

/* ------------------------------------------------------------------------ */
/* Section 2.A: exponent probabilities of N(0, sigma^2) and the top-7 table   */
/* ------------------------------------------------------------------------ */

/*
 * Probability that a value X ~ N(0, sigma^2) carries BF16 exponent field e.
 * A normal BF16 number with exponent field e (1..254) has magnitude in
 * [2^(e-127), 2^(e-126)); field 0 holds zero and the subnormals, |X| < 2^-126;
 * field 255 (Inf/NaN) never occurs for a finite Gaussian draw.
 *   P(a <= |X| < b) = erfc(a / (sigma*sqrt2)) - erfc(b / (sigma*sqrt2)).
 * The octave bounds are the exact powers of two (the BF16 rounding of values
 * just below a power of two is ignored: the pages give no rounding rule).
 */
int zco_exponent_probabilities(double sigma, double p[256]) {
    if (!(sigma > 0.0) || !isfinite(sigma)) return ZCO_ERR_INVALID_ARG;
    const double s = sigma * sqrt(2.0);
    p[0] = erf(ldexp(1.0, -126) / s);
    for (int e = 1; e <= 254; ++e) {
        double lo = ldexp(1.0, e - 127);
        double hi = ldexp(1.0, e - 126);
        p[e] = erfc(lo / s) - erfc(hi / s);
    }
    p[255] = 0.0;
    return ZCO_OK;
}

/*
 * The 7 exponent fields of largest weight w[e], returned in ascending order.
 * Ties between equal weights go to the smaller field.  Code k (1..7) stands
 * for exps[k-1].
 */
static void top7_ascending(const double w[256], uint8_t exps[7]) {
    int taken[256];
    memset(taken, 0, sizeof(taken));
    int chosen[7];
    for (int k = 0; k < 7; ++k) {
        int best = -1;
        for (int e = 0; e < 256; ++e) {
            if (taken[e]) continue;
            if (best < 0 || w[e] > w[best]) best = e; /* strict '>' keeps the smaller e on ties */
        }
        taken[best] = 1;
        chosen[k] = best;
    }
    /* ascending order: insertion sort of seven values */
    for (int i = 1; i < 7; ++i) {
        int v = chosen[i], j = i - 1;
        while (j >= 0 && chosen[j] > v) {
            chosen[j + 1] = chosen[j];
            --j;
        }
        chosen[j + 1] = v;
    }
    for (int k = 0; k < 7; ++k) exps[k] = (uint8_t)chosen[k];
}

/* The 7 most probable exponents of N(0, sigma^2) (section 2.A). */
int zco_plan_from_sigma(double sigma, uint8_t exps[7]) {
    double p[256];
    int rc = zco_exponent_probabilities(sigma, p);
    if (rc != ZCO_OK) return rc;
    top7_ascending(p, exps);
    return ZCO_OK;
}

/* A plan is usable when its seven exponents are strictly ascending. */
static int plan_is_valid(const uint8_t exps[7]) {
    for (int k = 1; k < 7; ++k)
        if (exps[k] <= exps[k - 1]) return 0;
    return 1;
}

/* ------------------------------------------------------------------------ */
/* Stream layout                                                             */
/* ------------------------------------------------------------------------ */

typedef struct {
    uint64_t n, words, groups;
    uint64_t off_sm, off_p0, off_p1, off_p2, off_tab, off_zp;
} zco_layout_t;

static zco_layout_t layout_of(uint64_t n) {
    zco_layout_t L;
    L.n = n;
    L.words = (n + 63) / 64;
    L.groups = (n + ZCO_GROUP - 1) / ZCO_GROUP;
    L.off_sm = ZCO_HEADER_BYTES;
    L.off_p0 = round_up_128(L.off_sm + n);
    L.off_p1 = L.off_p0 + round_up_128(8 * L.words);
    L.off_p2 = L.off_p1 + round_up_128(8 * L.words);
    L.off_tab = L.off_p2 + round_up_128(8 * L.words);
    L.off_zp = L.off_tab + round_up_128(4 * (L.groups + 1));
    return L;
}

/* Offsets of every section, for the tests: out[0..6] = off_sm, off_p0, off_p1,
 * off_p2, off_tab, off_zp, number of groups. */
void zco_layout(uint64_t n, uint64_t out[7]) {
    zco_layout_t L = layout_of(n);
    out[0] = L.off_sm;
    out[1] = L.off_p0;
    out[2] = L.off_p1;
    out[3] = L.off_p2;
    out[4] = L.off_tab;
    out[5] = L.off_zp;
    out[6] = L.groups;
}

/* Largest stream n elements can produce: every exponent on the zero-point path. */
uint64_t zco_max_bytes(uint64_t n) { return layout_of(n).off_zp + n; }

/* ------------------------------------------------------------------------ */
/* Section 2.B: encode                                                       */
/* ------------------------------------------------------------------------ */

/*
 * Encode n BF16 words (raw 16-bit patterns) with the seven exponents `exps`.
 * Writes total_bytes bytes of `out` (capacity `cap`) and returns the size.
 */
int zco_encode(const uint16_t *x, uint64_t n, const uint8_t exps[7], uint8_t *out, uint64_t cap,
               uint64_t *total_bytes) {
    if (!plan_is_valid(exps)) return ZCO_ERR_INVALID_ARG;
    if (n > 0xFFFFFFFFull) return ZCO_ERR_INVALID_ARG;
    zco_layout_t L = layout_of(n);
    if (cap < L.off_zp + n) return ZCO_ERR_CAPACITY;

    /* everything not written below is a zero pad */
    memset(out, 0, L.off_zp);

    uint8_t *sm = out + L.off_sm;
    uint8_t *plane[3] = {out + L.off_p0, out + L.off_p1, out + L.off_p2};
    uint8_t *tab = out + L.off_tab;
    uint8_t *zp = out + L.off_zp;
    uint64_t zp_count = 0;

    for (uint64_t i = 0; i < n; ++i) {
        uint16_t v = x[i];
        /* split: 1 sign bit, 8 exponent bits, 7 mantissa bits */
        unsigned sign = (v >> 15) & 1u;
        unsigned exponent = (v >> 7) & 0xFFu;
        unsigned mantissa = v & 0x7Fu;
        /* the sign+mantissa byte: sign in bit 7, mantissa in bits 6..0 */
        sm[i] = (uint8_t)((sign << 7) | mantissa);

        /* remap: position of the exponent among the seven, plus one; 0 if absent */
        unsigned code = 0;
        for (unsigned k = 0; k < 7; ++k)
            if (exps[k] == exponent) code = k + 1;

        /* three 1-bit arrays: plane b holds bit b of the code; element i is
           bit (i mod 8) of byte (i / 8), i.e. bit (i mod 64) of the
           little-endian 64-bit word (i / 64) */
        for (unsigned b = 0; b < 3; ++b)
            if ((code >> b) & 1u) plane[b][i / 8] |= (uint8_t)(1u << (i % 8));

        /* the zero-point table entry of a group is the number of zero-point
           values that precede its first element */
        if (i % ZCO_GROUP == 0) put_u32(tab + 4 * (i / ZCO_GROUP), (uint32_t)zp_count);

        /* zero-point code 000: the full exponent goes to the separate array */
        if (code == 0) zp[zp_count++] = (uint8_t)exponent;
    }
    put_u32(tab + 4 * L.groups, (uint32_t)zp_count);

    uint64_t total = L.off_zp + zp_count;
    put_u32(out + 0, ZCO_MAGIC);
    put_u16(out + 4, ZCO_VERSION);
    put_u16(out + 6, ZCO_HEADER_BYTES);
    put_u64(out + 8, n);
    put_u32(out + 16, ZCO_GROUP);
    put_u32(out + 20, (uint32_t)L.groups);
    for (int k = 0; k < 7; ++k) out[24 + k] = exps[k];
    out[31] = ZCO_MODE_CODED;
    put_u64(out + 32, zp_count);
    put_u64(out + 40, total);
    *total_bytes = total;
    return ZCO_OK;
}

/*
 * Encode with a raw fallback.  The pages describe no fallback; with many
 * zero-point values the coded stream grows past the 16 bits of the input
 * (each such value costs 8 + 3 + 8 bits).  Reading used here: the result is
 * whichever is smaller, the coded stream or the raw one; a tie keeps the
 * coded stream.  A raw stream has the same header with byte 31 ("mode") = 1
 * and total_bytes = 128 + 2n (exps and E still describe the coded form that
 * was not kept); the n BF16 words follow the header unchanged, little-endian.
 */
int zco_encode_fallback(const uint16_t *x, uint64_t n, const uint8_t exps[7], uint8_t *out, uint64_t cap,
                        uint64_t *total_bytes) {
    int rc = zco_encode(x, n, exps, out, cap, total_bytes);
    if (rc != ZCO_OK) return rc;
    const uint64_t raw_total = ZCO_HEADER_BYTES + 2 * n;
    if (*total_bytes > raw_total) {
        out[31] = ZCO_MODE_RAW;
        put_u64(out + 40, raw_total);
        for (uint64_t i = 0; i < n; ++i) put_u16(out + ZCO_HEADER_BYTES + 2 * i, x[i]);
        *total_bytes = raw_total;
    }
    return ZCO_OK;
}

/* ------------------------------------------------------------------------ */
/* Decode (strict: any field or pad that the encoder could not have written   */
/* is rejected before a single element is produced)                          */
/* ------------------------------------------------------------------------ */

static int bytes_are_zero(const uint8_t *p, uint64_t len) {
    for (uint64_t i = 0; i < len; ++i)
        if (p[i]) return 0;
    return 1;
}

static unsigned code_at(const uint8_t *const plane[3], uint64_t i) {
    unsigned c = 0;
    for (unsigned b = 0; b < 3; ++b) c |= (unsigned)((plane[b][i / 8] >> (i % 8)) & 1u) << b;
    return c;
}

int zco_decode(const uint8_t *in, uint64_t in_bytes, uint64_t n, uint16_t *x) {
    if (n > 0xFFFFFFFFull) return ZCO_ERR_INVALID_ARG;
    zco_layout_t L = layout_of(n);
    if (in_bytes < ZCO_HEADER_BYTES) return ZCO_ERR_CORRUPT;

    /* header */
    if (get_u32(in + 0) != ZCO_MAGIC) return ZCO_ERR_CORRUPT;
    if (get_u16(in + 4) != ZCO_VERSION) return ZCO_ERR_CORRUPT;
    if (get_u16(in + 6) != ZCO_HEADER_BYTES) return ZCO_ERR_CORRUPT;
    if (get_u64(in + 8) != n) return ZCO_ERR_CORRUPT;
    if (get_u32(in + 16) != ZCO_GROUP) return ZCO_ERR_CORRUPT;
    if (get_u32(in + 20) != L.groups) return ZCO_ERR_CORRUPT;
    uint8_t exps[7];
    for (int k = 0; k < 7; ++k) exps[k] = in[24 + k];
    if (!plan_is_valid(exps)) return ZCO_ERR_CORRUPT;
    const uint8_t mode = in[31];
    if (mode != ZCO_MODE_CODED && mode != ZCO_MODE_RAW) return ZCO_ERR_CORRUPT;
    uint64_t zp_count = get_u64(in + 32);
    uint64_t total = get_u64(in + 40);
    if (zp_count > n) return ZCO_ERR_CORRUPT;
    if (mode == ZCO_MODE_RAW) {
        /* raw fallback: the header, then the n words unchanged */
        if (total != ZCO_HEADER_BYTES + 2 * n) return ZCO_ERR_CORRUPT;
        if (total > in_bytes) return ZCO_ERR_CORRUPT;
        if (!bytes_are_zero(in + 48, ZCO_HEADER_BYTES - 48)) return ZCO_ERR_CORRUPT;
        for (uint64_t i = 0; i < n; ++i) x[i] = get_u16(in + ZCO_HEADER_BYTES + 2 * i);
        return ZCO_OK;
    }
    if (total != L.off_zp + zp_count) return ZCO_ERR_CORRUPT;
    if (total > in_bytes) return ZCO_ERR_CORRUPT;
    if (!bytes_are_zero(in + 48, ZCO_HEADER_BYTES - 48)) return ZCO_ERR_CORRUPT;

    const uint8_t *sm = in + L.off_sm;
    const uint8_t *plane[3] = {in + L.off_p0, in + L.off_p1, in + L.off_p2};
    const uint8_t *tab = in + L.off_tab;
    const uint8_t *zp = in + L.off_zp;

    /* pads: after SM, after every plane (including the bits past element n-1),
       after the table */
    if (!bytes_are_zero(sm + n, L.off_p0 - (L.off_sm + n))) return ZCO_ERR_CORRUPT;
    for (unsigned b = 0; b < 3; ++b) {
        uint64_t used = (n + 7) / 8;
        if (n % 8 && (plane[b][n / 8] >> (n % 8))) return ZCO_ERR_CORRUPT;
        if (!bytes_are_zero(plane[b] + used, (L.off_p1 - L.off_p0) - used)) return ZCO_ERR_CORRUPT;
    }
    if (!bytes_are_zero(tab + 4 * (L.groups + 1), (L.off_zp - L.off_tab) - 4 * (L.groups + 1)))
        return ZCO_ERR_CORRUPT;

    /* table: starts at 0, ends at E, and each group's step equals the number
       of zero-point codes inside that group */
    if (get_u32(tab) != 0) return ZCO_ERR_CORRUPT;
    if (get_u32(tab + 4 * L.groups) != zp_count) return ZCO_ERR_CORRUPT;
    for (uint64_t g = 0; g < L.groups; ++g) {
        uint64_t first = g * ZCO_GROUP;
        uint64_t last = first + ZCO_GROUP < n ? first + ZCO_GROUP : n;
        uint64_t zeros = 0;
        for (uint64_t i = first; i < last; ++i) zeros += code_at(plane, i) == 0;
        uint32_t a = get_u32(tab + 4 * g), b = get_u32(tab + 4 * (g + 1));
        if (b < a || (uint64_t)(b - a) != zeros) return ZCO_ERR_CORRUPT;
    }

    /* rebuild: exponent from the table of seven, or the next zero-point byte */
    uint64_t k = 0;
    for (uint64_t i = 0; i < n; ++i) {
        unsigned c = code_at(plane, i);
        unsigned exponent = c ? exps[c - 1] : zp[k++];
        unsigned sign = (sm[i] >> 7) & 1u;
        unsigned mantissa = sm[i] & 0x7Fu;
        x[i] = (uint16_t)((sign << 15) | (exponent << 7) | mantissa);
    }
    return ZCO_OK;
}

/* ------------------------------------------------------------------------ */
/* Local reduction of the reduce-scatter path (section 2.D: a reduce-scatter  */
/* may run as a zipped all-to-all followed by a local reduction)              */
/* ------------------------------------------------------------------------ */
/* Readings (the pages name the path only):
 *   - each of the k streams carries one peer's BF16 contribution to the same
 *     n elements; the receiver may also hold its own BF16 contribution
 *     (`local`, uncompressed, nullable);
 *   - per element the terms are added in IEEE single precision, in the order
 *     local, stream 0, stream 1, ..., each addition rounded to nearest-even;
 *     the first term enters exactly (no 0.0f + term, which would turn -0 into
 *     +0);
 *   - the float sum is rounded to BF16, nearest with ties to even; a NaN sum
 *     becomes the quiet NaN 0x7FC0.
 * A stream that fails strict decoding fails the whole reduction. */

static float bf16_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Nearest BF16 to a float: the two candidates are the float truncated to its
   upper 16 bits and the next BF16 away from zero; halfway goes to the one with
   an even last mantissa bit.  Overflow past the largest BF16 gives infinity. */
uint16_t zco_float_to_bf16(float f) {
    if (isnan(f)) return 0x7FC0u;
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lower = u >> 16, rest = u & 0xFFFFu;
    if (rest > 0x8000u || (rest == 0x8000u && (lower & 1u))) lower += 1;
    return (uint16_t)lower;
}

int zco_decode_reduce(const uint8_t *const *streams, const uint64_t *in_bytes, uint32_t k, uint64_t n,
                      const uint16_t *local, uint16_t *out) {
    if (n > 0xFFFFFFFFull || (k == 0 && !local)) return ZCO_ERR_INVALID_ARG;
    float *acc = (float *)malloc((n ? n : 1) * sizeof(float));
    uint16_t *term = (uint16_t *)malloc((n ? n : 1) * sizeof(uint16_t));
    if (!acc || !term) {
        free(acc);
        free(term);
        return ZCO_ERR_INVALID_ARG;
    }
    int first = 1;
    if (local) {
        for (uint64_t i = 0; i < n; ++i) acc[i] = bf16_to_float(local[i]);
        first = 0;
    }
    for (uint32_t s = 0; s < k; ++s) {
        int rc = zco_decode(streams[s], in_bytes[s], n, term);
        if (rc != ZCO_OK) {
            free(acc);
            free(term);
            return rc;
        }
        for (uint64_t i = 0; i < n; ++i) acc[i] = first ? bf16_to_float(term[i]) : acc[i] + bf16_to_float(term[i]);
        first = 0;
    }
    for (uint64_t i = 0; i < n; ++i) out[i] = zco_float_to_bf16(acc[i]);
    free(acc);
    free(term);
    return ZCO_OK;
}

/* ------------------------------------------------------------------------ */
/* Plan variants (section 2.A: the table of seven comes from sigma "instead   */
/* of costly online histogram construction or sorting"; both routes are      */
/* written out here so that they can be compared)                             */
/* ------------------------------------------------------------------------ */

/* Count of every exponent field in x. */
void zco_exponent_histogram(const uint16_t *x, uint64_t n, uint64_t hist[256]) {
    for (int e = 0; e < 256; ++e) hist[e] = 0;
    for (uint64_t i = 0; i < n; ++i) hist[(x[i] >> 7) & 0xFFu] += 1;
}

/* The seven most frequent exponent fields, ascending; equal counts go to the
   smaller field (so fields that never occur fill up from 0 when fewer than
   seven occur).  Counts below 2^53 convert to double exactly. */
int zco_plan_from_histogram(const uint64_t hist[256], uint8_t exps[7]) {
    double w[256];
    for (int e = 0; e < 256; ++e) w[e] = (double)hist[e];
    top7_ascending(w, exps);
    return ZCO_OK;
}

/* Sigma of a tensor for the closed-form plan.  Reading: the pages model the
   values as N(0, sigma^2); the estimate is the root mean square of the finite
   values (exponent field below 255), i.e. the maximum-likelihood sigma of a
   zero-mean Gaussian.  Squares of BF16 values are exact in double; the sum is
   taken in element order.  Returns 0 when no value is finite. */
double zco_estimate_sigma(const uint16_t *x, uint64_t n, uint64_t *finite) {
    double sum = 0.0;
    uint64_t m = 0;
    for (uint64_t i = 0; i < n; ++i) {
        if (((x[i] >> 7) & 0xFFu) == 0xFFu) continue;
        double v = (double)bf16_to_float(x[i]);
        sum += v * v;
        m += 1;
    }
    if (finite) *finite = m;
    return m ? sqrt(sum / (double)m) : 0.0;
}
