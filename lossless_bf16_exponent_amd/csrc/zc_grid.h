// Layout of the compress grid (host side): which blocks of one launch encode
// which spans, and where each segment's finalize blocks go.
//
// The grid is a sequence of pieces: the encoder blocks of a segment, or its
// finalize blocks.  Encoder pieces come in segment order.  A segment's
// finalize piece goes right after the first encoder piece that ends kFinLag or
// more encoder blocks past the end of its own encoder piece (by then its
// blocks have most likely finished, and its finalize work overlaps the
// encoding of later segments), else at the end of the grid.  Every finalize
// block thus comes after every encoder block it waits for; workgroups are
// dispatched in index order.
#pragma once

#include <stdint.h>

#include "zc_format.h"

namespace zc {

constexpr uint32_t kMaxSegments = 64;
constexpr uint32_t kMaxPieces = 2 * kMaxSegments;
constexpr uint8_t kPieceFinalize = 0x80;  // piece info: this bit (a finalize piece), plus the segment in bits 0..6
constexpr uint64_t kFinLag = 2048;         // about the number of blocks the device keeps in flight

struct GridPlan {
    uint32_t pieces;
    uint32_t piece_start[kMaxPieces + 1];  // first grid block of each piece; the last entry is the grid size
    uint8_t piece_info[kMaxPieces];
};

// Returns false when k is out of range or the grid would exceed 2^32 - 1 blocks.
inline bool plan_grid(const uint64_t *n, uint32_t k, GridPlan &g) {
    if (k == 0 || k > kMaxSegments) return false;
    uint64_t pos = 0, enc_done = 0;
    uint64_t enc_end[kMaxSegments];
    uint32_t next_fin = 0;
    g.pieces = 0;
    auto add_piece = [&](uint32_t info, uint64_t blocks) {
        g.piece_start[g.pieces] = (uint32_t)pos;
        g.piece_info[g.pieces] = (uint8_t)info;
        ++g.pieces;
        pos += blocks;
    };
    for (uint32_t i = 0; i < k; ++i) {
        const uint64_t nb = enc_blocks(n[i]);
        add_piece(i, nb);
        enc_done += nb;
        enc_end[i] = enc_done;
        while (next_fin < i && enc_done - enc_end[next_fin] >= kFinLag) {
            add_piece(kPieceFinalize | next_fin, fin_blocks(n[next_fin]));
            ++next_fin;
        }
        if (pos > 0xFFFFFFFFull) return false;
    }
    for (; next_fin < k; ++next_fin) add_piece(kPieceFinalize | next_fin, fin_blocks(n[next_fin]));
    if (pos > 0xFFFFFFFFull) return false;
    g.piece_start[g.pieces] = (uint32_t)pos;
    return true;
}

}  // namespace zc
