// Host check of the compress grid layout (zc_grid.h): for random and
// boundary batches, one unit and several units per block, every encoder span
// and every finalize run of every segment has exactly one place in the grid;
// a launch of at most kDirectMax encoder blocks is all direct (unless staged
// only is asked for), a longer one all staged; every unit comes after every
// unit it waits for -- in a lower block, or earlier in its own block: a
// finalize run after the encoder spans of its run and the segment's earlier
// runs, a direct span after the segment's earlier spans.  Built by
// tests/test_host.py; no GPU.
#include <cstdio>
#include <vector>

#include "zc_grid.h"

using namespace zc;

static uint64_t rng_state = 0x2545F4914F6CDD1Dull;
static uint64_t rnd() {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return rng_state;
}

static int failures = 0;
#define CHECK(cond)                                                                      \
    do {                                                                                 \
        if (!(cond)) {                                                                   \
            if (failures++ < 10) std::printf("FAIL line %d: %s\n", __LINE__, #cond);     \
        }                                                                                \
    } while (0)

// The device's view of grid block `flat`: which segment, which role, which
// units [index, end).
struct Role {
    uint32_t seg, kind;
    uint64_t index, end;
};

static Role role_of(const GridPlan &g, uint32_t flat, const std::vector<uint64_t> &n) {
    uint32_t p = 0;
    // linear: independent of the kernel's search
    while (p + 1 < g.pieces && (g.piece[p + 1] & kBlockMask) <= flat) ++p;
    const uint32_t w = g.piece[p];
    const uint32_t seg = w >> 26, kind = (w >> 24) & 3u;
    const uint64_t u0 = (uint64_t)g.first[p] + (uint64_t)(flat - (w & kBlockMask)) * g.mult;
    const uint64_t nb = seg < n.size() ? enc_blocks(n[seg]) : 0;
    if (kind == kPieceSample) return Role{(uint32_t)u0, kind, u0, u0 + 1};  // sampler of segment u0
    const uint64_t e = piece_end(kind, g.first[p], nb, g.chunk);
    return Role{seg, kind, u0, u0 + g.mult < e ? u0 + g.mult : e};
}

static void check_batch(const std::vector<uint64_t> &n, uint32_t mult = 1, bool staged_only = false,
                        bool sample = false) {
    GridPlan g;
    CHECK(plan_grid(n.data(), (uint32_t)n.size(), g, mult, staged_only, sample));
    CHECK(g.pieces <= kMaxPieces);
    const uint32_t total = g.piece[g.pieces];
    CHECK(total < kMaxGrid);
    const size_t k = n.size();
    std::vector<std::vector<int64_t>> enc_pos(k), fin_pos(k);
    std::vector<std::vector<int>> enc_kind(k);
    uint64_t all_spans = 0;
    for (size_t s = 0; s < k; ++s) {
        enc_pos[s].assign(enc_blocks(n[s]), -1);
        enc_kind[s].assign(enc_blocks(n[s]), -1);
        fin_pos[s].assign(g.direct ? 0 : ceil_div(enc_blocks(n[s]), kRun), -1);
        all_spans += enc_blocks(n[s]);
    }
    // a unit's place: its block, then its turn in the block (the order of execution)
    int64_t first_direct = -1;
    std::vector<int64_t> sampler(k, -1);
    int64_t first_other = -1;
    for (uint32_t flat = 0; flat < total; ++flat) {
        const Role r = role_of(g, flat, n);
        CHECK(r.seg < k && r.kind <= kPieceSample);
        CHECK(r.index < r.end && r.end - r.index <= mult);  // no empty block
        if (r.seg >= k) continue;
        if (r.kind == kPieceSample) {
            CHECK(sample && sampler[r.seg] == -1);  // one sampler per segment, only when asked for
            sampler[r.seg] = flat;
            continue;
        }
        if (first_other < 0) first_other = flat;
        for (uint64_t u = r.index; u < r.end; ++u) {
            const int64_t at = (int64_t)flat * 65536 + (int64_t)(u - r.index);
            if (r.kind == kPieceFinalize) {
                std::vector<int64_t> &v = fin_pos[r.seg];
                CHECK(u < v.size());
                if (u < v.size()) {
                    CHECK(v[u] == -1);  // each run once
                    v[u] = at;
                }
            } else {
                if (r.kind == kPieceDirect && first_direct < 0) first_direct = flat;
                std::vector<int64_t> &v = enc_pos[r.seg];
                CHECK(u < v.size());
                if (u < v.size()) {
                    CHECK(v[u] == -1);  // each span once
                    v[u] = at;
                    enc_kind[r.seg][u] = (int)r.kind;
                }
            }
        }
    }
    // the samplers, when asked for, open the grid: every block of a segment waits for its sampler
    for (size_t s = 0; s < k; ++s) CHECK(sample ? sampler[s] >= 0 && sampler[s] < first_other : sampler[s] < 0);
    // a launch that fits kDirectMax blocks is all direct, a longer one all staged
    const bool direct = all_spans <= kDirectMax && !staged_only;
    CHECK(direct == (first_direct >= 0) && direct == g.direct);
    for (size_t s = 0; s < k; ++s) {
        const uint64_t nb = enc_blocks(n[s]);
        for (uint64_t b = 0; b < nb; ++b) {
            CHECK(enc_pos[s][b] >= 0);
            CHECK(enc_kind[s][b] == (direct ? (int)kPieceDirect : (int)kPieceStaged));
        }
    }
    for (size_t s = 0; s < k; ++s) {
        const uint64_t nb = enc_blocks(n[s]);
        if (g.direct) {
            for (uint64_t b = 1; b < nb; ++b) CHECK(enc_pos[s][b] > enc_pos[s][b - 1]);  // earlier spans' words
            continue;
        }
        const uint64_t nr = ceil_div(nb, kRun);
        int64_t max_fin = -1;
        for (uint64_t r = 0; r < nr; ++r) {
            const int64_t at = fin_pos[s][r];
            CHECK(at >= 0);
            const uint64_t end = (r + 1) * kRun < nb ? (r + 1) * kRun : nb;
            for (uint64_t b = r * kRun; b < end; ++b) CHECK(enc_pos[s][b] < at);  // the spans of its run
            CHECK(at > max_fin);                                                  // earlier runs' words
            max_fin = at;
        }
    }
}

int main() {
    // single segments around the tail and chunk thresholds, with ragged tails
    const uint64_t tile = kEncSpan;
    const uint64_t singles[] = {0,           1,           8191,       8192,        8193,           tile * 31,
                                tile * 32 + 5, tile * 2047, tile * 2048, tile * 2049, tile * 2065 + 3, tile * 4096 + 77,
                                tile * 7168, tile * 40000 + 1, tile * 131072};
    for (uint64_t n : singles) {
        check_batch({n});
        check_batch({n}, 1, false, true);  // the fallback's first launch
        check_batch({n}, 16, true);        // the fallback's second launch
        check_batch({n}, 3, false);
    }
    // the gradient bucket and the all-to-all shapes, and random batches (some empty segments)
    check_batch(std::vector<uint64_t>(32, tile * 1024));
    check_batch(std::vector<uint64_t>(64, tile * 1024 * 64));  // every segment one chunk only after growing it
    check_batch(std::vector<uint64_t>(64, tile * 32));         // exactly kDirectMax blocks: direct
    check_batch(std::vector<uint64_t>(64, tile * 32 + 1));     // one block more per segment: staged
    check_batch(std::vector<uint64_t>(64, tile * 1024 * 64), 1, false, true);  // the piece table full
    for (int it = 0; it < 400; ++it) {
        const size_t k = 1 + rnd() % kMaxSegments;
        std::vector<uint64_t> n(k);
        for (auto &x : n) {
            const uint64_t r = rnd() % 8;
            x = r == 0 ? 0 : (r < 4 ? rnd() % (tile * 64) : rnd() % (tile * 6000));
        }
        check_batch(n);
        check_batch(n, 1, false, true);
        check_batch(n, 16, true);
        check_batch(n, 1 + (uint32_t)(rnd() % 20), (rnd() & 1) != 0);
    }
    // the largest segment is planned
    {
        GridPlan g;
        const uint64_t big[] = {0xFFFFFFFFull};
        CHECK(plan_grid(big, 1, g));
        const uint64_t nb = enc_blocks(big[0]);
        CHECK(g.piece[g.pieces] == nb + ceil_div(nb, kRun));
    }
    if (failures) {
        std::printf("%d failures\n", failures);
        return 1;
    }
    std::printf("grid layout ok\n");
    return 0;
}
