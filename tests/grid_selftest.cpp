// Host check of the compress grid layout (zc_grid.h): for random
// batches, every encoder span and every finalize block of every segment has
// exactly one grid block, and every finalize block comes after every block it
// waits for -- the encoder blocks of the spans up to the end of its run, the
// finalize blocks of the segment's earlier runs, and (for a segment's last
// finalize block) every other finalize block of the segment.  Built by
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

// The device's view of grid block `flat`: which segment, which role, which index.
struct Role {
    uint32_t seg;
    bool fin;
    uint64_t index;
};

static Role role_of(const GridPlan &g, uint32_t flat) {
    uint32_t p = 0;
    while (p + 1 < g.pieces && g.piece_start[p + 1] <= flat) ++p;  // linear: independent of the kernel's search
    const uint32_t info = g.piece_info[p];
    return Role{info & 0x7Fu, (info & kPieceFinalize) != 0, (uint64_t)(flat - g.piece_start[p])};
}

static void check_batch(const std::vector<uint64_t> &n) {
    GridPlan g;
    CHECK(plan_grid(n.data(), (uint32_t)n.size(), g));
    const uint32_t total = g.piece_start[g.pieces];
    const size_t k = n.size();
    std::vector<std::vector<int64_t>> enc_pos(k), fin_pos(k);
    for (size_t s = 0; s < k; ++s) {
        enc_pos[s].assign(enc_blocks(n[s]), -1);
        fin_pos[s].assign(fin_blocks(n[s]), -1);
    }
    for (uint32_t flat = 0; flat < total; ++flat) {
        const Role r = role_of(g, flat);
        CHECK(r.seg < k);
        std::vector<int64_t> &v = r.fin ? fin_pos[r.seg] : enc_pos[r.seg];
        CHECK(r.index < v.size());
        if (r.index < v.size()) {
            CHECK(v[r.index] == -1);  // each block once
            v[r.index] = flat;
        }
    }
    for (size_t s = 0; s < k; ++s) {
        const uint64_t nb = enc_blocks(n[s]), nf = fin_blocks(n[s]);
        const uint32_t run = fin_run(nb);
        for (uint64_t b = 0; b < nb; ++b) CHECK(enc_pos[s][b] >= 0);
        int64_t max_fin = -1;
        for (uint64_t j = 0; j < nf; ++j) {
            const int64_t at = fin_pos[s][j];
            CHECK(at >= 0);
            const uint64_t end = (j + 1) * run < nb ? (j + 1) * run : nb;
            for (uint64_t b = 0; b < end; ++b) CHECK(enc_pos[s][b] < at);  // spans up to the end of its run
            for (uint64_t i = 0; i < j; ++i) CHECK(fin_pos[s][i] < at);    // earlier runs' words
            if (j + 1 < nf) max_fin = at > max_fin ? at : max_fin;
        }
        CHECK(fin_pos[s][nf - 1] > max_fin);  // the last block waits for every other one
    }
}

int main() {
    // single segments around the interleaving thresholds, with ragged tails
    const uint64_t tile = kEncSpan;
    const uint64_t singles[] = {0, 1, 8191, 8192, 8193, tile * 31, tile * 32 + 5, tile * 2047, tile * 2048,
                                tile * 2049, tile * 4096 + 77, tile * 7168, tile * 40000 + 1};
    for (uint64_t n : singles) check_batch({n});
    // the gradient bucket shape and random batches (some empty segments)
    check_batch(std::vector<uint64_t>(32, tile * 1024));
    for (int it = 0; it < 300; ++it) {
        const size_t k = 1 + rnd() % kMaxSegments;
        std::vector<uint64_t> n(k);
        for (auto &x : n) {
            const uint64_t r = rnd() % 8;
            x = r == 0 ? 0 : (r < 4 ? rnd() % (tile * 64) : rnd() % (tile * 3000));
        }
        check_batch(n);
    }
    // the largest segment and a batch near the 2^32-block grid limit are planned
    {
        GridPlan g;
        const uint64_t big[] = {0xFFFFFFFFull};
        CHECK(plan_grid(big, 1, g));
        CHECK(g.piece_start[g.pieces] == enc_blocks(big[0]) + fin_blocks(big[0]));
    }
    if (failures) {
        std::printf("%d failures\n", failures);
        return 1;
    }
    std::printf("grid layout ok\n");
    return 0;
}
