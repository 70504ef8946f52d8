// Stream format constants and section offsets of the BF16 exponent codec.
//
// Format of one stream (see include/zc.h for the full table): a 128-byte
// header, the sign+mantissa bytes, three 1-bit code planes, a table of
// zero-point counts per 4096-element group and the zero-point exponent bytes.
// Every section starts on a 128-byte boundary: the ZipCCL explainer pages
// ("ZipCCL: Efficient Lossless Data Compression of Communication Collectives
// for Accelerating LLM Training", section 2.C) pad data blocks to 128-byte
// boundaries so that every global access is a whole, coalesced 128-byte
// transaction.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define ZC_HD __host__ __device__ __forceinline__
#else
#define ZC_HD static inline
#endif

namespace zc {

constexpr uint32_t kMagic = 0x3143435Au;  // "ZCC1"
constexpr uint16_t kVersion = 1;
constexpr uint32_t kHeaderBytes = 128;
constexpr uint32_t kGroup = 4096;  // elements per zero-point table entry
constexpr uint64_t kMaxElems = 0xFFFFFFFFull;
constexpr uint32_t kModeCoded = 0;  // header byte 31: the coded layout
constexpr uint32_t kModeRaw = 1;    // header byte 31: the raw fallback (header, then the n values)

// Encoder / decoder tiling (not part of the format; the stream does not depend
// on it).  A lane owns 8 consecutive elements (one 16-byte load) per step; a
// wave64 step covers 512 elements; a 256-thread block makes kSteps steps.
constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kSteps = 4;
constexpr uint32_t kTile = kThreads * 8 * kSteps;  // 8192 elements
constexpr uint32_t kGroupsPerTile = kTile / kGroup;
static_assert(kTile % kGroup == 0, "a tile holds whole groups");

// The encoder gives each block a span of kEncSubTiles consecutive tiles.
#ifndef ZC_ENC_SUBTILES
#define ZC_ENC_SUBTILES 1
#endif
constexpr int kEncSubTiles = ZC_ENC_SUBTILES;
constexpr uint32_t kEncSpan = kTile * kEncSubTiles;
constexpr int kEncGroups = (int)(kEncSpan / kGroup);

ZC_HD uint64_t enc_blocks(uint64_t n) {
    const uint64_t b = (n + kEncSpan - 1) / kEncSpan;
    return b ? b : 1;
}

// The decoder gives each block a span of kDecSubTiles consecutive tiles.
#ifndef ZC_DEC_SUBTILES
#define ZC_DEC_SUBTILES 2
#endif
constexpr int kDecSubTiles = ZC_DEC_SUBTILES;
constexpr uint32_t kDecSpan = kTile * kDecSubTiles;
constexpr int kDecGroups = (int)(kDecSpan / kGroup);

ZC_HD uint64_t dec_blocks(uint64_t n) {
    const uint64_t b = (n + kDecSpan - 1) / kDecSpan;
    return b ? b : 1;
}

ZC_HD uint64_t align128(uint64_t x) { return (x + 127u) & ~uint64_t(127u); }

struct Layout {
    uint64_t n;
    uint64_t plane_bytes;  // 8 * ceil(n / 64), the section padded to 128
    uint64_t groups;       // NG
    uint64_t off_p0, off_p1, off_p2, off_tab, off_zp;
    uint64_t off_scratch;  // encoder scratch behind the largest stream
    uint64_t tiles;        // encoder tiles (at least one, so n = 0 still writes a header)
};

ZC_HD Layout layout_for(uint64_t n) {
    Layout L;
    L.n = n;
    L.plane_bytes = align128(8 * ((n + 63) / 64));
    L.groups = (n + kGroup - 1) / kGroup;
    L.off_p0 = align128(kHeaderBytes + n);
    L.off_p1 = L.off_p0 + L.plane_bytes;
    L.off_p2 = L.off_p1 + L.plane_bytes;
    L.off_tab = L.off_p2 + L.plane_bytes;
    L.off_zp = L.off_tab + align128(4 * (L.groups + 1));
    L.off_scratch = align128(L.off_zp + n);
    uint64_t t = (n + kTile - 1) / kTile;
    L.tiles = t ? t : 1;
    return L;
}

// Finalize blocks: each one completes a run of consecutive encoder spans.  A
// run has at least kFinRunMin spans, more when a segment would otherwise need
// over kFinMaxBlocks finalize blocks.
constexpr uint32_t kFinRunMin = 16;
constexpr uint32_t kFinMaxBlocks = 1024;
ZC_HD uint32_t fin_run(uint64_t nb) {
    const uint64_t r = (nb + kFinMaxBlocks - 1) / kFinMaxBlocks;
    return (uint32_t)(r > kFinRunMin ? r : kFinRunMin);
}
ZC_HD uint64_t fin_blocks(uint64_t n) {
    const uint64_t nb = enc_blocks(n);
    const uint32_t r = fin_run(nb);
    return (nb + r - 1) / r;
}
constexpr uint32_t kFinRunMax = (uint32_t)((((kMaxElems + kEncSpan - 1) / kEncSpan) + kFinMaxBlocks - 1) / kFinMaxBlocks);

// Encoder scratch, at off_scratch (behind the largest possible stream):
//   span words  16 B per encoder span: zero-point counts of its two groups
//   run words   16 B per finalize block: zero-point total of its run
//   done words  16 B per finalize block: the block has finished its waits
//   staging     kEncSpan B per encoder span: its zero-point bytes, in order
// Every word carries the 64-bit token of the call that wrote it, so words
// left by an earlier call (or any other old contents) never pass for fresh.
constexpr uint32_t kWordBytes = 16;
struct Scratch {
    uint64_t span_words, run_words, done_words, staging, bytes;  // offsets from off_scratch, total size
};
ZC_HD Scratch scratch_for(uint64_t n) {
    const uint64_t nb = enc_blocks(n), nf = fin_blocks(n);
    Scratch S;
    S.span_words = 0;
    S.run_words = align128(kWordBytes * nb);
    S.done_words = S.run_words + align128(kWordBytes * nf);
    S.staging = S.done_words + align128(kWordBytes * nf);
    S.bytes = S.staging + nb * (uint64_t)kEncSpan;
    return S;
}

}  // namespace zc
