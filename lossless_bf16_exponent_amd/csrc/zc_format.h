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
#include <hip/hip_runtime.h>
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

// The decoder gives each block a span of one or two consecutive tiles, the
// same for every segment of a launch: one tile when the launch decodes at
// least kDecNarrowMin values or at most kDecNarrowMax, two in between.
// (Measured on MI355X: one-tile spans decode long launches 3-4 % faster once
// the device has settled, and launches too small to fill the device up to
// 20 % faster; in between, 58.7 Mi values for one, they were 3 % slower.)
// Test builds move the thresholds so that either form takes every launch.
#ifndef ZC_DEC_NARROW_MIN
#define ZC_DEC_NARROW_MIN (1ull << 27)
#endif
#ifndef ZC_DEC_NARROW_MAX
#define ZC_DEC_NARROW_MAX (1ull << 23)
#endif
constexpr uint64_t kDecNarrowMin = ZC_DEC_NARROW_MIN;
constexpr uint64_t kDecNarrowMax = ZC_DEC_NARROW_MAX;
constexpr int kDecWideTiles = 2;
constexpr uint32_t kDecRawSpan = kTile * kDecWideTiles;  // values per block of the raw-only decoder

// Blocks for n values in spans of `span` values (at least one, so that n = 0
// still checks its header).
ZC_HD uint64_t dec_blocks(uint64_t n, uint32_t span) {
    const uint64_t b = (n + span - 1) / span;
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

// Compress work split (not part of the format).  Encoder spans are coded in
// one of two modes:
//   * staged (a launch longer than the device holds at once): the block stages
//     its zero-point bytes in scratch and leaves; a finalize block later places
//     the bytes of a run of kRun consecutive spans;
//   * direct (a launch of at most kDirectMax encoder blocks, all resident at
//     once): the block finds its place in the zero-point array itself and
//     writes its bytes there.
// Prefix sums of zero-point counts come from a hierarchy of words that blocks
// publish for each other: a span word per span; in staged mode a run word per
// finalize run and a chunk word per kChunkRuns runs; in direct mode a group
// word per kGroupSpans spans.
constexpr uint32_t kRun = 16;
constexpr uint32_t kChunkRuns = 64;
constexpr uint32_t kChunkSpans = kRun * kChunkRuns;  // 1024
constexpr uint32_t kGroupSpans = 64;
constexpr uint32_t kDirectMax = 2048;  // about the number of blocks the device holds at once
constexpr uint32_t kMaxDirectGroups = (kDirectMax + kGroupSpans - 1) / kGroupSpans;

ZC_HD uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

// Encoder scratch, at off_scratch (behind the largest possible stream), sized
// for either mode:
//   decision      raw fallback: the first pass's guess, raw or coded
//   status        raw fallback: what the second pass still has to do
//   epoch         8 bytes, no token: a counter the segment's header writer
//                 advances at the end of each call's first launch
//   failed        set by a block of the segment whose wait ran out
//   span words    one per encoder span: zero-point counts of its two groups
//   run words     one per run: zero-point count of the run
//   chunk words   one per chunk: zero-point count of its runs
//   group words   one per group of direct spans: their zero-point count
//   staging       kEncSpan B per encoder span: its zero-point bytes, in order
// Every word carries the 64-bit token of the launch that wrote it, so words
// left by an earlier launch (or any other old contents) never pass for fresh.
// A launch's token is the call's token from the host mixed with the epoch, so
// that it also changes between replays of a captured graph, which repeat the
// host's arguments.
constexpr uint32_t kWordBytes = 16;
struct Scratch {
    uint64_t decision, status, epoch, failed, span_words, run_words, chunk_words, group_words, staging,
        bytes;  // offsets from off_scratch, total size
};
ZC_HD Scratch scratch_for(uint64_t n) {
    const uint64_t nb = enc_blocks(n), nr = ceil_div(nb, kRun), nc = ceil_div(nr, kChunkRuns);
    const uint64_t ng = ceil_div(nb, kGroupSpans);
    Scratch S;
    S.decision = 0;
    S.status = kWordBytes;
    S.epoch = 2 * kWordBytes;
    S.failed = 3 * kWordBytes;
    S.span_words = align128(4 * kWordBytes);
    S.run_words = S.span_words + align128(kWordBytes * nb);
    S.chunk_words = S.run_words + align128(kWordBytes * nr);
    S.group_words = S.chunk_words + align128(kWordBytes * nc);
    S.staging = S.group_words + align128(kWordBytes * ng);
    S.bytes = S.staging + nb * (uint64_t)kEncSpan;
    return S;
}

}  // namespace zc
