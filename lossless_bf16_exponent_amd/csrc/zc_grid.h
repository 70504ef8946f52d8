// Layout of the compress grid (host side): which blocks of one launch encode
// which spans, in which mode, and where the finalize blocks go.
//
// A launch of at most kDirectMax encoder blocks (all of them resident at
// once) is coded in direct mode: every block finds its own place in the
// zero-point array and writes its bytes there.  A longer launch is staged:
// while the device is saturated, a round trip between blocks costs as much as
// a data load under that load (measured: about 5 us), so no encoder block
// waits; finalize blocks place the staged bytes instead.  Each segment's
// spans are cut into chunks of `chunk` spans (a multiple of kChunkSpans; one
// chunk for most segments, several for a long one, as the piece table
// allows).  A chunk's finalize blocks (one per run of kRun spans) go right
// after the first encoder chunk that ends kFinLag or more encoder blocks past
// the end of their own chunk (by then its blocks have most likely finished,
// and the finalize work overlaps later encoding), or at the end of the grid.
//
// Every block waits only for blocks placed before it: a finalize block for
// the encoder blocks of its run and for the finalize blocks of earlier runs of
// its segment; a direct block for earlier direct blocks of its segment.
// Workgroups are dispatched in index order, so every block waited for has been
// dispatched first.
//
// A grid may give each block `mult` consecutive units (spans of an encoder
// piece, runs of a finalize piece) instead of one, taken in order: a unit
// then also waits for units of its own block, all of them done before it.
// The raw fallback's second launch does so, since most of its blocks have
// nothing to do and a launch pays per block.
#pragma once

#include <stdint.h>

#include "zc_format.h"

namespace zc {

constexpr uint32_t kMaxSegments = 64;
// Pieces: at most two per segment (a staged chunk and its finalize blocks)
// once the chunk size has grown to hold each segment; one per segment in
// direct mode; and the sampler piece of a launch that guesses.
constexpr uint32_t kMaxPieces = 2 * kMaxSegments + 1;
constexpr uint32_t kPieceStaged = 0, kPieceDirect = 1, kPieceFinalize = 2, kPieceSample = 3;
constexpr uint64_t kFinLag = 2048;          // about the number of blocks the device keeps in flight
constexpr uint32_t kMaxGrid = 1u << 24;     // grid blocks; piece starts keep 24 bits
constexpr uint32_t kBlockMask = kMaxGrid - 1;

// piece word: bits 0..23 the piece's first grid block, bits 24..25 its kind,
// bits 26..31 its segment.
inline uint32_t piece_word(uint64_t start, uint32_t kind, uint32_t seg) {
    return (uint32_t)start | (kind << 24) | (seg << 26);
}

struct GridPlan {
    uint32_t pieces;
    uint32_t piece[kMaxPieces + 1];  // piece words; entry [pieces] holds the grid size
    uint32_t first[kMaxPieces];      // first span (encoder pieces) or first run (finalize pieces) in the segment
    bool direct;                     // the launch is coded in direct mode
    uint64_t chunk;                  // spans per staged chunk
    uint32_t mult;                   // units (spans or runs) per block
};

// The units a piece covers end at (exclusive): a direct piece at the
// segment's last span, a staged piece at its chunk's end, a finalize piece
// at the last run of its chunk.  nb: the segment's spans; first: the piece's
// first unit.
ZC_HD uint64_t piece_end(uint32_t kind, uint64_t first, uint64_t nb, uint64_t chunk) {
    if (kind == kPieceDirect) return nb;
    if (kind == kPieceStaged) return first + chunk < nb ? first + chunk : nb;
    const uint64_t f = first * kRun;  // the chunk's first span
    return ceil_div(f + chunk < nb ? f + chunk : nb, kRun);
}

// Returns false when k is out of range or the grid would reach kMaxGrid blocks.
// staged_only: never direct (the fallback's second launch, whose blocks take
// several units).  sample: the grid opens with one sampler block per segment
// (the raw fallback's first launch: every block of a guessing segment waits
// for its sampler).
inline bool plan_grid(const uint64_t *n, uint32_t k, GridPlan &g, uint32_t mult = 1, bool staged_only = false,
                      bool sample = false) {
    if (k == 0 || k > kMaxSegments) return false;
    uint64_t nb[kMaxSegments], total = 0;
    for (uint32_t i = 0; i < k; ++i) {
        nb[i] = enc_blocks(n[i]);
        total += nb[i];
    }
    uint64_t grid = 0;
    g.pieces = 0;
    auto add = [&](uint32_t kind, uint32_t seg, uint64_t first, uint64_t units) {
        g.piece[g.pieces] = piece_word(grid, kind, seg);
        g.first[g.pieces] = (uint32_t)first;
        ++g.pieces;
        grid += ceil_div(units, mult);
        return grid < kMaxGrid;
    };
    if (mult == 0 || (sample && mult != 1)) return false;
    g.mult = mult;
    if (sample) add(kPieceSample, 0, 0, k);
    g.direct = total <= kDirectMax && !staged_only;
    g.chunk = kChunkSpans;
    if (g.direct) {
        for (uint32_t i = 0; i < k; ++i)
            if (!add(kPieceDirect, i, 0, nb[i])) return false;
        g.piece[g.pieces] = (uint32_t)grid;
        return true;
    }
    // chunk size: the smallest of 1024, 2048, ... spans that fits the piece table
    auto pieces_for = [&](uint64_t c) {
        uint64_t p = sample ? 1 : 0;
        for (uint32_t i = 0; i < k; ++i) p += 2 * ceil_div(nb[i], c);
        return p;
    };
    while (pieces_for(g.chunk) > kMaxPieces) g.chunk *= 2;

    struct Pending {
        uint32_t seg, first_run, runs;
        uint64_t ready;  // encoder blocks emitted when it may go
    };
    Pending queue[kMaxPieces];
    uint32_t qh = 0, qt = 0;
    uint64_t enc_done = 0;
    for (uint32_t i = 0; i < k; ++i) {
        for (uint64_t f = 0; f < nb[i]; f += g.chunk) {
            const uint64_t cnt = nb[i] - f < g.chunk ? nb[i] - f : g.chunk;
            if (!add(kPieceStaged, i, f, cnt)) return false;
            enc_done += ceil_div(cnt, mult);
            const uint64_t r0 = f / kRun, r1 = ceil_div(f + cnt, kRun);
            queue[qt++] = Pending{i, (uint32_t)r0, (uint32_t)(r1 - r0), enc_done + kFinLag};
            while (qh < qt && queue[qh].ready <= enc_done) {
                if (!add(kPieceFinalize, queue[qh].seg, queue[qh].first_run, queue[qh].runs)) return false;
                ++qh;
            }
        }
    }
    for (; qh < qt; ++qh)
        if (!add(kPieceFinalize, queue[qh].seg, queue[qh].first_run, queue[qh].runs)) return false;
    g.piece[g.pieces] = (uint32_t)grid;
    return true;
}

}  // namespace zc
