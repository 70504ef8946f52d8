// Compress kernels and their C ABI: the BF16 exponent-coding codec for MI355X
// (gfx950).
//
// Method: the ZipCCL explainer pages ("ZipCCL: Efficient Lossless Data
// Compression of Communication Collectives for Accelerating LLM Training"),
// technical summary section 2.B: split every BF16 value into a sign+mantissa
// byte and its exponent; an exponent among the seven of the table becomes a
// 3-bit code 001..111, any other gets 000 and its full byte is appended to a
// separate zero-point array.  Section 2.C: 128-byte aligned blocks for
// coalesced 128-bit accesses, the 3-bit codes as three 1-bit arrays.
//
// Design on gfx950 (pure HBM-bandwidth path, no MFMA):
//   * a 256-thread block codes one 8192-element span; a lane loads 8 values
//     with one 128-bit load per step, so every wave-wide load or store is a
//     contiguous 1 KiB (input), 512 B (sign+mantissa) or 64 B (plane) run;
//   * codes and bit planes come from dword-wide byte shuffles (zc_lane.h), and
//     the per-lane plane bytes are regrouped through LDS into whole dwords per
//     plane before they are stored;
//   * zero-point bytes are placed by an exclusive scan across the tensor.  In
//     a launch longer than the device holds at once, encoder blocks never wait:
//     each leaves its zero-point count (a span word) and its zero-point bytes
//     staged in the segment's scratch (in the call's workspace, or behind the
//     stream in the output buffer).  Finalize blocks of the same launch,
//     placed about a device's worth of blocks behind the spans they complete,
//     sum the counts through a hierarchy of run and chunk words, fill the
//     table and move the staged bytes to their place.  A launch the device
//     holds at once is coded in direct mode: each block finds its own place
//     and writes its bytes there, with no staging.  Blocks wait only for
//     blocks of the same launch with lower indices, which workgroup dispatch
//     in index order has started first; every wait is bounded, and a call
//     whose wait runs out still ends, with a zero magic in its header and a
//     stream size of 0: a block whose wait runs out marks its segment as
//     failed, and the segment's last block, which writes the header, reads
//     the mark once its own waits have passed.  Those waits depend, directly
//     or through other words, on a word from every other block of the
//     segment, so by then every word that any block of the segment waits for
//     has been published and a wait still pending ends at its next poll
//     (zc_grid.h places the roles; the scratch words are described below,
//     with the reasons the handshakes are device-scope accesses and not
//     release/acquire pairs);
//   * under the raw fallback the first launch guesses each long segment's
//     form from a sample and a second launch completes wrong guesses.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cstring>
#include <random>

#include "zc.h"
#include "zc_device.h"
#include "zc_format.h"
#include "zc_grid.h"
#include "zc_host.h"
#include "zc_lane.h"

namespace zc {

// Timeline of a compress launch, in an instrumented build only (ZC_TIMELINE,
// the bench's libzc_timeline.so; the codec library compiles none of it):
// thread 0 of each block records the real-time clock (100 MHz) at four points
// of its role, and the role itself.  Stamp 0: the block starts; 1: an encoder
// block's first pass is done (loads, codes, counts), a finalize block has its
// run's span words; 2: a staged encoder block has stored its zero-point bytes
// and seen them acknowledged, a direct one knows its offset, a finalize block
// has landed its run's bytes and knows their offset; 3: the block ends.
#ifdef ZC_TIMELINE
constexpr uint32_t kTimelineBlocks = 1u << 20;
constexpr uint32_t kTimelineWords = 5;  // four stamps and the role
__device__ unsigned long long zc_timeline[kTimelineBlocks * kTimelineWords];
__device__ __forceinline__ void stamp(uint32_t point) {
    if (threadIdx.x == 0 && blockIdx.x < kTimelineBlocks)
        zc_timeline[blockIdx.x * kTimelineWords + point] = __builtin_amdgcn_s_memrealtime();
}
__device__ __forceinline__ void stamp_role(uint32_t kind, uint32_t seg, uint32_t unit) {
    if (threadIdx.x == 0 && blockIdx.x < kTimelineBlocks)
        zc_timeline[blockIdx.x * kTimelineWords + 4] = kind | (seg << 2) | ((unsigned long long)unit << 8);
}
#else
__device__ __forceinline__ void stamp(uint32_t) {}
__device__ __forceinline__ void stamp_role(uint32_t, uint32_t, uint32_t) {}
#endif

// ---------------------------------------------------------------------------
// kernel arguments (passed by value; at most ZC_MAX_BATCH segments)
// ---------------------------------------------------------------------------

struct EncSeg {
    const uint16_t *in;
    uint8_t *out;
    unsigned long long *out_bytes;
    uint32_t n;
    uint8_t exps[7];
    uint8_t flags;     // kSegTable, kSegRawOk
    uint32_t ws_off;   // with a workspace: the segment's scratch at ws + 256 * ws_off
};
static_assert(sizeof(EncSeg) == 40, "compact kernel arguments");
constexpr uint8_t kSegTable = 1;  // codes from a 256-byte LDS table (else: the window's saturating arithmetic)
constexpr uint8_t kSegRawOk = 2;  // the plan allows the raw fallback

// The compress grid is a sequence of pieces (zc_grid.h).
static_assert(kMaxSegments == ZC_MAX_BATCH, "one segment per batch entry");

struct EncArgs {
    uint32_t k;
    uint32_t pieces;
    uint32_t tok_lo, tok_hi;  // the launch's token (scratch words of other launches never match it)
    uint32_t prev_lo, prev_hi;  // the fallback's second launch: the token of the call's first launch
    uint32_t advance;           // 1: each segment's header writer advances the segment's epoch
    uint32_t mult;            // units (spans or runs) per block (zc_grid.h)
    uint32_t chunk;           // spans per staged chunk
    uint8_t *ws;              // the call's workspace, or null: each segment's scratch behind its stream
    EncSeg seg[ZC_MAX_BATCH];
    // Piece words (zc_grid.h: first grid block, kind, segment; the last entry
    // holds the grid size) and each piece's first span or run.  Words, not
    // bytes: with a byte array the compiler once shared an address base + p
    // between a byte read and a word read, giving a scalar load a base that is
    // not 4-byte aligned, which the scalar unit does not honour.
    uint32_t piece[kMaxPieces + 1];
    uint32_t first[kMaxPieces];
};
// Kept within the conventional 4 KiB kernel-argument budget, counting up to
// 256 bytes of the runtime's hidden arguments.
static_assert(sizeof(EncArgs) + 256 <= 4096, "compress arguments fit the kernarg segment");

// A segment's encoder scratch: in the call's workspace, or behind the
// largest stream in its own output buffer.
__device__ __forceinline__ uint8_t *seg_scratch(const EncArgs &a, const EncSeg &sg) {
    return a.ws ? a.ws + 256ull * sg.ws_off : sg.out + layout_for(sg.n).off_scratch;
}

// The piece holding grid block `flat` (piece words keep the block in their low 24 bits).
__device__ __forceinline__ uint32_t find_piece(const EncArgs &a, uint32_t flat) {
    return count_at_or_below<kMaxPieces + 1>(a.piece, a.pieces, flat, kBlockMask);
}

// ---------------------------------------------------------------------------
// scratch words shared between the blocks of one compress launch
// ---------------------------------------------------------------------------

// Each word is 16 bytes: two u64 halves, each holding half of the call's
// 64-bit token in bits 63..32 and the same 32-bit payload in bits 31..0.  A
// reader accepts a word only when both token halves match and both payloads
// agree, so old contents pass for fresh with probability about 2^-64.
//
// Ordering between blocks.  The writer and the reader may sit on different
// XCDs, whose L2 caches are not coherent with each other.  Every access to
// memory that one block writes and another block of the same launch reads (the
// words and the staged zero-point bytes) is a device-scope (agent) access:
// relaxed agent-scope atomics for the words, which gfx950 issues with the sc1
// cache policy, 16-byte buffer stores with that policy for the staged bytes
// and direct-to-LDS loads with it to read them back.  An sc1 store writes through the
// L2 to the device's coherence point and its vmcnt completion means it has
// reached that point; an sc1 load is served from that point, never from a
// stale line of the reader's L2.  So a writer that stores data with sc1, waits
// for vmcnt(0) and then stores a word, and a reader that loads the word and
// only then issues its sc1 loads of the data (their addresses depend on the
// word's payload), see the data the word announces.  This is what a
// release/acquire pair would give, without its L2 maintenance: the compiler
// implements an agent-scope release as buffer_wbl2 sc1 (write back every
// dirty L2 line) and an acquire as buffer_inv sc1 (invalidate the L2), which
// only data accessed without sc1 needs.  Measured with release stores and
// acquire loads on the words instead, compress of the 256 Mi-value bucket took
// 3,058 us instead of 155 us.  Words that announce no data (counts, done
// flags) need no wait before their store.
struct Token {
    uint32_t lo, hi;
};

__device__ __forceinline__ void put_word(uint8_t *w, Token t, uint32_t payload) {
    uint64_t *p = reinterpret_cast<uint64_t *>(w);
    __hip_atomic_store(p, ((uint64_t)t.lo << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p + 1, ((uint64_t)t.hi << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A word's two halves as loaded, checked against token t.
__device__ __forceinline__ bool word_valid(uint64_t a, uint64_t b, Token t, uint32_t &payload) {
    payload = (uint32_t)a;
    return (uint32_t)(a >> 32) == t.lo && (uint32_t)(b >> 32) == t.hi && (uint32_t)a == (uint32_t)b;
}
__device__ __forceinline__ void load_word(const uint8_t *w, uint64_t &a, uint64_t &b) {
    uint64_t *p = reinterpret_cast<uint64_t *>(const_cast<uint8_t *>(w));
    a = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    b = __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool get_word(const uint8_t *w, Token t, uint32_t &payload) {
    uint64_t a, b;
    load_word(w, a, b);
    return word_valid(a, b, t, payload);
}

// The segment's epoch word, read by every block of a launch before
// it publishes or polls anything.  The segment's header writer advances it at
// the end of a call's first launch, once its own waits have passed: those
// depend on a word from every other block of the segment, each published after
// its block read the epoch.  So within a launch the
// word does not change while anyone reads it, and a load that may hit the L2
// serves: the value a reader needs was written by an earlier launch on the
// stream, which the kernel boundary makes visible.  (A device-scope load from
// every block of the launch, all to one line, cost 2-4 us per call.)  It is a
// vector load (a workgroup-scope atomic, which the compiler never turns into a
// scalar load): a scalar load would be waited for with every later wait for
// scalar or LDS results, which complete out of order.
__device__ __forceinline__ uint64_t *epoch_word(const EncArgs &args, const EncSeg &sg) {
    return reinterpret_cast<uint64_t *>(seg_scratch(args, sg) + scratch_for(sg.n).epoch);
}
__device__ __forceinline__ uint64_t read_epoch(const EncArgs &args, const EncSeg &sg) {
    return __hip_atomic_load(epoch_word(args, sg), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// A launch's token for a segment: the call's token from the host mixed with
// the segment's epoch.  A replay of a captured graph repeats the host's token
// but not the epoch, so its words never pass for the previous replay's.
__device__ __forceinline__ Token mix_token(uint32_t lo, uint32_t hi, uint64_t epoch) {
    return Token{lo ^ (uint32_t)epoch, hi ^ (uint32_t)(epoch >> 32)};
}
__device__ __forceinline__ Token launch_token(const EncArgs &args, const EncSeg &sg) {
    return mix_token(args.tok_lo, args.tok_hi, read_epoch(args, sg));
}

// Staged zero-point bytes move between blocks with the same cache policy as
// the atomics above (sc1: written through to the device's coherence point),
// 16 bytes per lane through a buffer resource that covers one staging slot:
// a wave's store is 1 KiB of whole lines.  (With two 8-byte atomic stores per
// 16 bytes, each instruction wrote every other 8 bytes of its lines, written
// through as partial lines: the escape-heavy 1 Gi-value stress input then
// compressed in 1,156 us instead of 970 us.)
constexpr int kCachePolicySc1 = 16;      // the sc1 bit of a memory instruction's cache policy
constexpr int kBufferDword3 = 0x00020000;  // raw buffer resource word 3 (gfx9 family: untyped, no swizzle)

__device__ __forceinline__ void put_staged16(__amdgpu_buffer_rsrc_t slot, uint32_t off, uint4 v) {
    const u32x4 d = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(d, slot, (int)off, 0, kCachePolicySc1);
}

// Waits poll at most this often before the call is given up (with s_sleep
// between polls this is well over a second, far beyond the longest encode).
// Only a dispatch that did not follow workgroup order could reach it; the
// kernel then still ends, the header gets a zero magic (every decoder rejects
// the stream) and the stream size reads 0.  A test build sets ZC_SPIN_LIMIT to
// 0 so that every wait gives up at once.
#ifndef ZC_SPIN_LIMIT
#define ZC_SPIN_LIMIT (1u << 20)
#endif
constexpr uint32_t kSpinLimit = ZC_SPIN_LIMIT;
// A test build sets ZC_FAIL_OTHERS to 1: every finalize block and direct span
// other than a segment's header writer then acts as if one of its waits had
// run out, while the header writer's own waits pass, so that the failure mark
// alone must keep the stream from being marked valid.  Such a block sets the
// mark, and waits for it to be acknowledged, before it publishes any word, as
// a block that gave up would have done before the words the header writer
// waits for appeared.
#ifndef ZC_FAIL_OTHERS
#define ZC_FAIL_OTHERS 0
#endif

// Thread tid polls words addr(i), i = tid + kThreads q (q < Q, i < count),
// until every one carries the token.  Payloads of valid words land in pay[q]
// (0 for indices at or past count).  done: bit q set when the caller has
// already found word q valid, its payload in pay[q].  Returns false on timeout.
template <int Q, typename Addr>
__device__ __forceinline__ bool poll_list(uint32_t count, Addr addr, Token t, uint32_t (&pay)[Q],
                                          uint32_t done = 0) {
    const uint32_t i0 = threadIdx.x;
    uint32_t pend = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        if (!(done >> q & 1u)) pay[q] = 0;
        if (i0 + kThreads * q < count && !(done >> q & 1u)) pend |= 1u << q;
    }
    for (uint32_t it = 0; pend; ++it) {
        if (it == kSpinLimit) return false;
        if (it) __builtin_amdgcn_s_sleep(2);
        bool got[Q];
        uint32_t v[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) got[q] = (pend >> q & 1u) && get_word(addr(i0 + kThreads * q), t, v[q]);
#pragma unroll
        for (int q = 0; q < Q; ++q)
            if (got[q]) {
                pay[q] = v[q];
                pend &= ~(1u << q);
            }
    }
    return true;
}

// A block whose wait ran out marks its segment's launch as failed (thread 0;
// ok is block-uniform).  The header writer reads the mark before it writes the
// header: a given-up wait of any block of the segment invalidates the stream.
__device__ __forceinline__ void mark_failed(uint8_t *scratch, const Scratch &S, Token tok, bool ok) {
    if (!ok && threadIdx.x == 0) put_word(scratch + S.failed, tok, 1u);
}

// The same over words base[0 .. count).
template <int Q>
__device__ __forceinline__ bool poll_words(const uint8_t *base, uint32_t count, Token t, uint32_t (&pay)[Q],
                                           uint32_t done = 0) {
    return poll_list<Q>(count, [base](uint32_t i) { return base + (uint64_t)kWordBytes * i; }, t, pay, done);
}

// Sum of v over the block (every thread gets it); red: kWaves words of LDS.
// Starts and ends with a barrier, so red may be reused right after.
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t *red) {
    const uint32_t w = wave_sum(v);
    __syncthreads();
    if (__lane_id() == 0) red[threadIdx.x / kWave] = w;
    __syncthreads();
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) t += red[i];
    __syncthreads();
    return t;
}

// ---------------------------------------------------------------------------
// compress: one launch, encoder blocks first, then finalize blocks
// ---------------------------------------------------------------------------

// One step of one lane: 8 consecutive values (16 bytes) starting at `base`.
struct Step {
    uint32_t d[4];
    uint32_t vmask;  // bit k set when value k is below n
};

__device__ __forceinline__ Step load_step(const uint16_t *in, uint64_t base, uint64_t n) {
    Step st;
    if (base + 8 <= n) {
        const uint4 v = load_stream16(in + base);
        st.d[0] = v.x;
        st.d[1] = v.y;
        st.d[2] = v.z;
        st.d[3] = v.w;
        st.vmask = 0xFFu;
    } else {
        uint32_t w4[4] = {0, 0, 0, 0};
        const uint32_t have = base < n ? (uint32_t)(n - base) : 0u;
        for (uint32_t i = 0; i < have; ++i) w4[i / 2] |= (uint32_t)in[base + i] << (16 * (i % 2));
        st.d[0] = w4[0];
        st.d[1] = w4[1];
        st.d[2] = w4[2];
        st.d[3] = w4[3];
        st.vmask = (1u << have) - 1u;
    }
    return st;
}

// LDS of a compress block; the encoder and finalize roles share it.
struct EncShared {
    uint32_t planes[kTile / 8];              // per 8-value group: plane bytes 0, 1, 2
    __align__(16) uint8_t zp[kEncSpan + 16];  // the span's zero-point bytes, in order (+ slack for reads past them)
    uint8_t code[256];                        // table mode: exponent -> code
    uint32_t wave_total[2][kWaves];
    uint32_t group[kEncGroups];               // zero-points per 4096-value group of the span
    uint32_t red[kWaves];
};
// LDS landing zone of the copy: batches of spans whose staged bytes (rounded
// up to 16) fit; any single span (at most kEncSpan bytes) does.
constexpr uint32_t kLandBytes = 12288;
static_assert(kLandBytes >= kEncSpan, "one span always lands");
struct FinShared {
    __align__(16) uint8_t land[kLandBytes + 48];  // landed staged bytes (+ slack for reads past a span)
    uint32_t pre[kRun + 1];     // zero-points of the run before each of its spans
    uint32_t land16[kRun + 1];  // 16-byte units of the run's spans before each span
    uint32_t g0[kRun];          // zero-points in the first group of each span
    uint32_t red[kWaves];
};
union CompressShared {
    EncShared e;
    FinShared f;
};
static_assert(kEncGroups == 2, "a span word holds the counts of two groups");
static_assert(kRun <= kWave, "a run's spans are scanned by one wave");
static_assert(kGroupSpans - 1 + kMaxDirectGroups <= kThreads, "a direct block polls its words in one round");

// Copy of staged zero-point bytes to the stream, in two phases.  Landing:
// the staged bytes of a batch of spans come into an LDS landing zone with
// direct global->LDS loads (16 bytes per lane, agent-scope), so every load of
// the batch is in flight at once and holds no registers.  Writing: a span's T
// bytes go to stream offset dst_off (any alignment); they cover destination
// dwords 0 .. ndw-1 counted from dst_off rounded down to 4, and destination
// dword k takes source bytes 4k - r .. 4k - r + 3 (r = dst_off mod 4): a
// byte-aligned window over source dwords k-1 and k of the landed copy.  A wave
// writes 128 destination dwords per round (lane l: dwords 2l, 2l + 1); dwords
// shared with the neighbouring spans get byte stores.
// Writes several small spans at once: a group of 16 lanes per span, each lane
// 8 consecutive destination dwords per round (128 per span-round).  Same
// destination bytes and byte-exact edges as write_span; sources: the span's
// landed copy (the zone has slack past every span).
__device__ __forceinline__ void write_span_group(uint8_t *zp, uint64_t dst_off, const uint8_t *land, uint32_t T,
                                                 uint32_t gl) {
    if (T == 0) return;
    const uint32_t r = (uint32_t)(dst_off & 3u);
    uint8_t *const dst = zp + (dst_off - r);
    const uint32_t ndw = (r + T + 3) / 4;
    const uint32_t *const w = reinterpret_cast<const uint32_t *>(land);
    for (uint32_t k0 = 8u * gl; k0 < ndw; k0 += 128u) {
        uint32_t src[9];  // source dwords k0 - 1 .. k0 + 7
        src[0] = k0 ? w[k0 - 1] : 0u;
        const uint4 a = *reinterpret_cast<const uint4 *>(w + k0), b = *reinterpret_cast<const uint4 *>(w + k0 + 4);
        src[1] = a.x; src[2] = a.y; src[3] = a.z; src[4] = a.w;
        src[5] = b.x; src[6] = b.y; src[7] = b.z; src[8] = b.w;
        const int64_t bk = (int64_t)4 * k0 - r;  // source index of byte 0 of dword k0
        if (k0 + 8 <= ndw && bk >= 0 && bk + 32 <= (int64_t)T) {
            // all 8 dwords inside the span: two 16-byte stores, streamed out of the L2
            uint32_t d[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) d[i] = r ? __builtin_amdgcn_alignbyte(src[i + 1], src[i], 4 - r) : src[i + 1];
            __builtin_nontemporal_store(u32x4a4{d[0], d[1], d[2], d[3]}, reinterpret_cast<u32x4a4 *>(dst + 4u * k0));
            __builtin_nontemporal_store(u32x4a4{d[4], d[5], d[6], d[7]},
                                        reinterpret_cast<u32x4a4 *>(dst + 4u * k0 + 16u));
            continue;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t m = k0 + (uint32_t)i;
            if (m >= ndw) break;
            const uint32_t d = r ? __builtin_amdgcn_alignbyte(src[i + 1], src[i], 4 - r) : src[i + 1];
            const int64_t b0 = (int64_t)4 * m - r;  // source index of the dword's byte 0
            if (b0 >= 0 && b0 + 4 <= (int64_t)T) {
                *reinterpret_cast<uint32_t *>(dst + 4u * m) = d;
            } else {
                for (int j = 0; j < 4; ++j)
                    if (b0 + j >= 0 && b0 + j < (int64_t)T) dst[4u * m + j] = (uint8_t)(d >> (8 * j));
            }
        }
    }
}


// Chunks c0, c0 + stride, ... of kWave units each (the waves of a block share
// a span's chunks, so one large span is not left to a single wave).
__device__ __forceinline__ void land_span(const uint8_t *src, uint32_t units, uint8_t *land, int lane, uint32_t c0,
                                          uint32_t stride) {
    for (uint32_t u0 = kWave * c0; u0 < units; u0 += kWave * stride) {
        if (u0 + (uint32_t)lane < units)
            __builtin_amdgcn_global_load_lds((global_void *)(src + 16u * (u0 + (uint32_t)lane)),
                                             (lds_void *)(land + 16u * u0), 16, 0, kCachePolicySc1);
    }
}

// Rounds c0, c0 + stride, ... of 2 * kWave destination dwords each.
__device__ __forceinline__ uint32_t span_dwords(uint64_t dst_off, uint32_t T) {
    return T ? ((uint32_t)(dst_off & 3u) + T + 3) / 4 : 0u;
}
__device__ __forceinline__ void write_span(uint8_t *zp, uint64_t dst_off, const uint8_t *land, uint32_t T, int lane,
                                           uint32_t c0, uint32_t stride) {
    if (T == 0) return;
    const uint32_t r = (uint32_t)(dst_off & 3u);
    uint8_t *const dst = zp + (dst_off - r);
    const uint32_t ndw = (r + T + 3) / 4;
    const uint32_t *const w = reinterpret_cast<const uint32_t *>(land);
    for (uint32_t k0 = 2 * kWave * c0; k0 < ndw; k0 += 2 * kWave * stride) {
        const uint32_t k = k0 + 2u * (uint32_t)lane;
        if (k >= ndw) break;
        // source dwords k-1 .. k+1 (the landing zone has slack past every span)
        const uint32_t sm1 = k ? w[k - 1] : 0u, s0 = w[k], s1 = w[k + 1];
        const uint32_t d0 = r ? __builtin_amdgcn_alignbyte(s0, sm1, 4 - r) : s0;
        const uint32_t d1 = r ? __builtin_amdgcn_alignbyte(s1, s0, 4 - r) : s1;
        const int64_t bk = (int64_t)4 * k - r;  // source index of byte 0 of dword k
        if (k + 1 < ndw && bk >= 0 && bk + 8 <= (int64_t)T) {
            // both dwords inside the span: one 8-byte store (a wave writes 512
            // contiguous bytes), streamed out of the L2
            __builtin_nontemporal_store(u32x2a4{d0, d1}, reinterpret_cast<u32x2a4 *>(dst + 4u * k));
            continue;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t m = k + h, d = h ? d1 : d0;
            if (m >= ndw) continue;
            const int64_t b0 = (int64_t)4 * m - r;  // source index of the dword's byte 0
            if (b0 >= 0 && b0 + 4 <= (int64_t)T) {
                *reinterpret_cast<uint32_t *>(dst + 4u * m) = d;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (b0 + j >= 0 && b0 + j < (int64_t)T) dst[4u * m + j] = (uint8_t)(d >> (8 * j));
            }
        }
    }
}


// Raw fallback (ZC_PLAN_RAW_FALLBACK).  The stream is raw when coding makes it
// larger: off_zp + E > 128 + 2n, which only the exact zero-point count E
// decides.  The call's first launch guesses, for each flagged segment long
// enough to sample: a sampler block at the front of the grid counts the
// zero-points of a sample spread over the segment and publishes its guess.
// The segment's blocks issue their loads, then read the guess (long
// published by then), and encoder blocks write
// either the coded sections or the raw copy of their span, counting the
// zero-points either way, and the segment's header writer applies the exact
// rule and leaves a status word.  The call's second launch, over the flagged
// segments only, completes what the first left: it copies the payload of a
// segment that was coded but came out raw, and codes a segment that was
// guessed raw but came out coded.  The stream never depends on the guess; a
// wrong guess costs the second pass over that segment.
constexpr uint32_t kSpecMinSpans = 64;    // shorter flagged segments are coded first, never guessed raw
constexpr uint32_t kSampleChunks = 1024;  // 8-value chunks the guess samples
enum : uint32_t { kModeCodedPass = 0, kModeSpecRaw = 1, kModeCopyRaw = 2, kModeSkip = 3, kModeAbort = 4 };
constexpr uint32_t kDecideRaw = 1, kDecideCoded = 2;
constexpr uint32_t kStatusFinal = 1, kStatusNeedRaw = 2, kStatusNeedCoded = 3;
#ifndef ZC_GUESS
#define ZC_GUESS 0  // test builds: 1 guesses raw, 2 guesses coded, for every flagged segment
#endif

__device__ __forceinline__ bool guesses(const EncSeg &sg) {
    return (sg.flags & kSegRawOk) &&
           (ZC_GUESS != 0 ? sg.n > 0 : enc_blocks(sg.n) >= (uint64_t)kSpecMinSpans);
}

// Second launch: what the first left for this segment (read once: the first
// launch has ended).  A segment without a status word of the first launch
// (given up) needs nothing.
__device__ __forceinline__ uint32_t second_pass_mode(const EncArgs &args, const EncSeg &sg) {
    const uint64_t e = read_epoch(args, sg);
    uint64_t a, b;
    load_word(seg_scratch(args, sg) + scratch_for(sg.n).status, a, b);  // in flight with the epoch
    // the first launch advanced the epoch once: its token used the one before
    const Token prev = mix_token(args.prev_lo, args.prev_hi, e - 1u);
    uint32_t st = 0;
    if (!word_valid(a, b, prev, st)) return kModeSkip;
    return st == kStatusNeedRaw ? kModeCopyRaw : (st == kStatusNeedCoded ? kModeCodedPass : kModeSkip);
}

// First launch, a block of a guessing segment: the guess (uniform), or
// kModeAbort when the wait for it gives up.
__device__ __forceinline__ uint32_t await_guess(const uint8_t *scratch, const Scratch &S, Token tok,
                                                uint32_t *red) {
    uint32_t d[1] = {0};
    bool ok = poll_words<1>(scratch + S.decision, 1, tok, d);
    ok = __syncthreads_and(ok);
    const uint32_t g = block_sum(d[0], red);  // thread 0's payload, to every thread
    return !ok ? kModeAbort : (g == kDecideRaw ? kModeSpecRaw : kModeCodedPass);
}

// Codes of the 8 values of one 16-byte chunk, as plane bytes (bits of values
// at or past n cleared by vmask).
__device__ __forceinline__ uint32_t chunk_planes(const uint32_t *d, uint32_t vmask, bool table, uint32_t base_hi,
                                                 const uint8_t *code) {
    const uint32_t t0 = exponent_high(d[0]), t1 = exponent_high(d[1]);
    const uint32_t t2 = exponent_high(d[2]), t3 = exponent_high(d[3]);
    uint32_t c_lo, c_hi;
    if (!table) {
        c_lo = window_codes4(t0, t1, base_hi);
        c_hi = window_codes4(t2, t3, base_hi);
    } else {
        const uint32_t e0 = exponents4(t0, t1), e1 = exponents4(t2, t3);
        c_lo = c_hi = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            c_lo |= (uint32_t)code[(e0 >> (8 * k)) & 0xFFu] << (8 * k);
            c_hi |= (uint32_t)code[(e1 >> (8 * k)) & 0xFFu] << (8 * k);
        }
    }
    return codes_to_planes(c_lo, c_hi) & (vmask * 0x010101u);
}

// The guess for a segment (first launch): zero-points among kSampleChunks
// chunks of 8 values spread evenly over the segment; raw when their share
// exceeds the break-even share (a sample of 8192 values has a standard error
// under 0.6 points).  Both wrong guesses cost about the same (a raw copy and a
// coded pass either way), so the estimate is taken as it is.
__device__ __forceinline__ uint32_t sample_guess(const EncSeg &sg, const Layout &L, bool table, uint32_t base_hi,
                                                 const uint8_t *code, uint32_t *red) {
    if (ZC_GUESS == 1) return kDecideRaw;
    if (ZC_GUESS == 2) return kDecideCoded;
    const uint64_t n = sg.n, chunks = n / 8;  // n >= kSpecMinSpans * kEncSpan: every sampled chunk is whole
    Step st[kSampleChunks / kThreads];
#pragma unroll
    for (uint32_t q = 0; q < kSampleChunks / kThreads; ++q) {
        const uint64_t j = threadIdx.x + kThreads * q;
        st[q] = load_step(sg.in, 8 * (j * chunks / kSampleChunks), n);
    }
    uint32_t z = 0;
#pragma unroll
    for (uint32_t q = 0; q < kSampleChunks / kThreads; ++q)
        z += __builtin_popcount(zero_point_mask(chunk_planes(st[q].d, st[q].vmask, table, base_hi, code)) &
                                st[q].vmask);
    const uint64_t zs = block_sum(z, red);
    const uint64_t S = 8ull * kSampleChunks, T = kHeaderBytes + 2 * n - L.off_zp;  // raw iff E > T
    return zs * n > S * T ? kDecideRaw : kDecideCoded;
}

// The n - span0 (at most kEncSpan) input values of a span behind the header
// (the raw payload), 16 bytes per lane and step.
__device__ __forceinline__ void copy_span_raw(const uint16_t *in, uint8_t *out, uint64_t span0, uint64_t n) {
    uint16_t *dst = reinterpret_cast<uint16_t *>(out + kHeaderBytes);
    constexpr uint32_t kPer = kEncSpan / (8 * kThreads);  // 16-byte units per lane of a whole span
    if (span0 + kEncSpan <= n) {  // every load in flight, then every store
        uint4 q[kPer];
#pragma unroll
        for (uint32_t i = 0; i < kPer; ++i) q[i] = load_stream16(in + span0 + 8u * (threadIdx.x + kThreads * i));
#pragma unroll
        for (uint32_t i = 0; i < kPer; ++i)
            store_stream16(dst + span0 + 8u * (threadIdx.x + kThreads * i), q[i].x, q[i].y, q[i].z, q[i].w);
        return;
    }
    const uint64_t v1 = min(span0 + kEncSpan, n), full = span0 + ((v1 - span0) & ~uint64_t(7));
    for (uint64_t v = span0 + 8u * threadIdx.x; v < full; v += 8u * kThreads) {
        const uint4 q = load_stream16(in + v);
        store_stream16(dst + v, q.x, q.y, q.z, q.w);
    }
    for (uint64_t v = full + threadIdx.x; v < v1; v += kThreads) dst[v] = in[v];
}

// The header, the table's last entry and the stream size of a segment with E
// zero-points.  ok = false (a wait given up somewhere in the segment) leaves a
// zero magic, which every decoder rejects, and a stream size of 0.  Raw
// fallback (first launch, kFb): the exact rule decides the form, and the
// segment's status word tells the second launch what is left: nothing, the
// raw payload (a coded pass that came out raw: the header already says raw),
// or the coded pass (a raw guess that came out coded: the header stays
// invalid until then).
template <bool kFb>
__device__ __forceinline__ void write_header(const EncArgs &args, const EncSeg &sg, const Layout &L, uint64_t E,
                                             bool ok, bool guessed_raw, Token tok) {
    const int tid = threadIdx.x;
    const uint64_t n = sg.n;
    uint8_t *const out = sg.out;
    const uint64_t raw_total = kHeaderBytes + 2 * n;
    const bool raw = kFb && (sg.flags & kSegRawOk) && L.off_zp + E > raw_total;
    // the stream is complete now (a coded pass that stays coded, a raw guess
    // that comes out raw), complete once the second launch has copied the
    // payload (coded pass, raw outcome), or left to the second launch entirely
    // (raw guess, coded outcome: the header stays invalid until then)
    const uint32_t status = !guessed_raw ? (raw ? kStatusNeedRaw : kStatusFinal)
                                         : (raw ? kStatusFinal : kStatusNeedCoded);
    const bool valid = ok && status != kStatusNeedCoded;
    const uint64_t total = raw ? raw_total : L.off_zp + E;
    if (valid && !raw && tid == 0) reinterpret_cast<uint32_t *>(out + L.off_tab)[L.groups] = (uint32_t)E;
    if (tid < 32) {
        uint32_t w = 0;
        switch (tid) {
            case 0: w = valid ? kMagic : 0u; break;
            case 1: w = (uint32_t)kVersion | (kHeaderBytes << 16); break;
            case 2: w = (uint32_t)n; break;
            case 3: w = (uint32_t)(n >> 32); break;
            case 4: w = kGroup; break;
            case 5: w = (uint32_t)L.groups; break;
            case 6: w = sg.exps[0] | (sg.exps[1] << 8) | (sg.exps[2] << 16) | ((uint32_t)sg.exps[3] << 24); break;
            case 7: w = sg.exps[4] | (sg.exps[5] << 8) | (sg.exps[6] << 16) | ((raw ? kModeRaw : kModeCoded) << 24); break;
            case 8: w = (uint32_t)E; break;
            case 9: w = (uint32_t)(E >> 32); break;
            case 10: w = (uint32_t)total; break;
            case 11: w = (uint32_t)(total >> 32); break;
            default: break;
        }
        reinterpret_cast<uint32_t *>(out)[tid] = w;
    }
    if (tid == 0 && sg.out_bytes) *sg.out_bytes = valid ? total : 0ull;
    if (kFb && ok && tid == 0 && (sg.flags & kSegRawOk))
        put_word(seg_scratch(args, sg) + scratch_for(n).status, tok, status);
    // the epoch this launch read (its token without the host's part), plus one
    if (args.advance && tid == 0)
        __hip_atomic_store(epoch_word(args, sg),
                           (((uint64_t)(tok.hi ^ args.tok_hi) << 32) | (tok.lo ^ args.tok_lo)) + 1u,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Direct role (every block of a launch that the device holds at once;
// zc_grid.h), in two steps.  As soon as the span's counts are known (before
// the zero-point bytes are collected) the block publishes its span word; the
// last span of each group of kGroupSpans spans then sums its group's span
// words and publishes the group word, so that no group word waits for another
// one.  Once its bytes are collected, the block finds the zero-points before
// its span: those of earlier groups through their group words and of the
// earlier spans of its own group through their span words, and writes its
// table entries and its zero-point bytes (from LDS) in place: nothing is
// staged.  The segment's last span then writes the header, unless the
// segment's failure mark is set: the group words it has read exist only once
// every span word of their groups does, so every other span's waits are for
// words already published.
struct DirectState {
    uint32_t sib;  // zero-points of the group's spans before b (the group's last span only)
    bool ok;
};
__device__ __forceinline__ DirectState direct_publish(const EncArgs &args, uint32_t s, uint32_t b, uint32_t c0,
                                                      uint32_t c1, Token tok, EncShared &sh) {
    const int tid = threadIdx.x;
    const EncSeg &sg = args.seg[s];
    const uint64_t n = sg.n;
    const Scratch S = scratch_for(n);
    const uint32_t nb = (uint32_t)enc_blocks(n);
    uint8_t *const scratch = seg_scratch(args, sg);
    const uint32_t g = b / kGroupSpans, g0 = g * kGroupSpans;  // g0: the group's first span
    const bool group_last = b % kGroupSpans == kGroupSpans - 1 || b + 1 == nb;
    if (ZC_FAIL_OTHERS && b + 1 < nb) {
        mark_failed(scratch, S, tok, false);
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    // a count announces no data: no wait before it
    if (tid == 0) put_word(scratch + S.span_words + (uint64_t)kWordBytes * b, tok, c0 | (c1 << 16));
    DirectState st{0u, true};
    if (group_last) {
        uint32_t sp[1];
        st.ok = poll_words<1>(scratch + S.span_words + (uint64_t)kWordBytes * g0, b - g0, tok, sp);
        st.ok = __syncthreads_and(st.ok);
        st.sib = block_sum((sp[0] & 0xFFFFu) + (sp[0] >> 16), sh.red);
        if (st.ok && tid == 0) put_word(scratch + S.group_words + (uint64_t)kWordBytes * g, tok, st.sib + c0 + c1);
    }
    return st;
}

template <bool kFb>
__device__ __forceinline__ void direct_finish(const EncArgs &args, uint32_t s, uint32_t b, uint32_t T, uint32_t c0,
                                              uint32_t c1, bool raw, DirectState st, Token tok, EncShared &sh) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const EncSeg &sg = args.seg[s];
    const uint64_t n = sg.n;
    const Layout L = layout_for(n);
    const Scratch S = scratch_for(n);
    const uint32_t nb = (uint32_t)enc_blocks(n);
    uint8_t *const out = sg.out;
    uint8_t *const scratch = seg_scratch(args, sg);
    const uint8_t *const span_w = scratch + S.span_words;
    const uint8_t *const group_w = scratch + S.group_words;
    const uint32_t g = b / kGroupSpans, g0 = g * kGroupSpans;
    const bool group_last = b % kGroupSpans == kGroupSpans - 1 || b + 1 == nb;
    bool ok = st.ok && !(ZC_FAIL_OTHERS && b + 1 < nb);
    const uint32_t sib = st.sib;
    // a raw guess places nothing: only the header writer needs its offset
    if (raw && b + 1 < nb) {
        mark_failed(scratch, S, tok, ok);
        return;
    }
    // the group's earlier spans (unless summed above) and the earlier groups
    const uint32_t nsib = group_last ? 0u : b - g0;
    uint32_t pay[1] = {0};
    if (ok)
        ok = poll_list<1>(
            nsib + g,
            [&](uint32_t i) {
                return i < nsib ? span_w + (uint64_t)kWordBytes * (g0 + i)
                                : group_w + (uint64_t)kWordBytes * (i - nsib);
            },
            tok, pay);
    ok = __syncthreads_and(ok);
    mark_failed(scratch, S, tok, ok);
    // the header writer: the failure mark, read once its own waits have passed
    // (in flight while it places its bytes)
    uint64_t fa = 0, fb = 0;
    if (b + 1 == nb) load_word(scratch + S.failed, fa, fb);
    const uint32_t mine = (uint32_t)tid < nsib ? (pay[0] & 0xFFFFu) + (pay[0] >> 16) : pay[0];
    const uint32_t P = sib + block_sum(mine, sh.red);
    stamp(2);

    if (ok && !raw) {
        uint32_t *const tab = reinterpret_cast<uint32_t *>(out + L.off_tab);
        const uint64_t gi = (uint64_t)b * kEncGroups;
        if (tid == 0 && gi < L.groups) tab[gi] = P;
        if (tid == 1 && gi + 1 < L.groups) tab[gi + 1] = P + c0;
        write_span(out + L.off_zp, P, sh.zp, T, lane, (uint32_t)wave, kWaves);
    }
    if (b + 1 < nb) return;
    uint32_t f;
    if (word_valid(fa, fb, tok, f)) ok = false;
    ok = __syncthreads_and(ok);
    write_header<kFb>(args, sg, L, (uint64_t)P + c0 + c1, ok, raw, tok);
}

// Encoder role under a raw guess: the span's loaded values go behind the
// header unchanged (the raw payload) and only their zero-points are counted,
// for the exact rule: waves 0 and 1 hold the span's first 4096-value group,
// waves 2 and 3 the second.
__device__ __forceinline__ void raw_span(const EncArgs &args, uint32_t s, uint32_t b, bool direct,
                                         const Step (&in)[kEncSubTiles][kSteps], bool table, uint32_t base_hi,
                                         Token tok, EncShared &sh) {
    static_assert(kEncSubTiles == 1 && kWaves == 4, "a span is one tile, two waves per group");
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const EncSeg &sg = args.seg[s];
    const uint64_t n = sg.n, span0 = (uint64_t)b * kEncSpan;
    uint16_t *const dst = reinterpret_cast<uint16_t *>(sg.out + kHeaderBytes);
    uint32_t z = 0;
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
        const uint64_t base = span0 + 512u * (uint32_t)(wave * kSteps + u) + 8u * (uint32_t)lane;
        const Step &st = in[0][u];
        z += __builtin_popcount(zero_point_mask(chunk_planes(st.d, st.vmask, table, base_hi, sh.code)) & st.vmask);
        if (st.vmask == 0xFFu) {
            store_stream16(dst + base, st.d[0], st.d[1], st.d[2], st.d[3]);
        } else {
#pragma unroll
            for (uint32_t i = 0; i < 8; ++i)  // constant indices keep st.d in registers
                if (st.vmask >> i & 1u) dst[base + i] = (uint16_t)(st.d[i / 2] >> (16 * (i % 2)));
        }
    }
    z = wave_sum(z);
    if (lane == 0) sh.red[wave] = z;
    __syncthreads();
    const uint32_t c0 = sh.red[0] + sh.red[1], c1 = sh.red[2] + sh.red[3];
    if (direct) {
        direct_finish<true>(args, s, b, 0, c0, c1, true, direct_publish(args, s, b, c0, c1, tok, sh), tok, sh);
        return;
    }
    // a count announces no data: no wait before the span word
    if (tid == 0) {
        const Scratch S = scratch_for(n);
        put_word(seg_scratch(args, sg) + S.span_words + (uint64_t)kWordBytes * b, tok, c0 | (c1 << 16));
    }
}

// Encoder role.  A block codes kEncSubTiles consecutive 8192-value sub-tiles
// (its span).  All loads of the span are issued up front.  Phase A turns every
// step into sign+mantissa bytes (stored at once), exponent bytes and plane
// bytes; phase B ranks the zero-point values, regroups and stores the planes
// and collects the zero-point bytes in LDS.  A staged span then stores its
// zero-point bytes to its staging slot, waits until every store of the block
// has completed and publishes its span word for the finalize blocks; a direct
// span places its bytes itself (direct_place).
template <bool kFb>
__device__ __forceinline__ void encode_span(const EncArgs &args, uint32_t s, uint32_t b, bool direct,
                                            EncShared &sh) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const EncSeg &sg = args.seg[s];  // b: block (span) index inside the segment
    const uint64_t n = sg.n;
    const Layout L = layout_for(n);
    const uint64_t blocks = enc_blocks(n);
    const bool table = (sg.flags & kSegTable) != 0;
    const uint64_t span0 = (uint64_t)b * kEncSpan;
    uint8_t *const out = sg.out;
    uint8_t *const scratch = seg_scratch(args, sg);
    const Scratch S = scratch_for(n);

    if (table) {
        uint32_t c = 0;
#pragma unroll
        for (int k = 0; k < 7; ++k) c = (sg.exps[k] == (uint32_t)tid) ? (uint32_t)(k + 1) : c;
        sh.code[tid] = (uint8_t)c;
    }
    const uint32_t wbase = (uint32_t)sg.exps[0] - 1u;  // window mode only (exps[0] >= 1)
    const uint32_t base_hi = (wbase << 8) | (wbase << 24);

    // ---- what this launch does with the span (raw fallback)
    uint32_t mode = kModeCodedPass;
    const bool guessing = kFb && guesses(sg);

    // the token: right ahead of the span's loads, which complete in order, so
    // that waiting for the first of them covers it
    const Token tok = launch_token(args, sg);

    // ---- every load of the span in flight at once
    Step in[kEncSubTiles][kSteps];
#pragma unroll
    for (int sub = 0; sub < kEncSubTiles; ++sub)
#pragma unroll
        for (int u = 0; u < kSteps; ++u)
            in[sub][u] = load_step(sg.in, span0 + (uint64_t)sub * kTile + 512u * (uint32_t)(wave * kSteps + u) +
                                              8u * (uint32_t)lane, n);
    if (kFb && guessing) {
        mode = await_guess(scratch, S, tok, sh.red);  // its barriers also cover sh.code
        if (mode == kModeAbort) {
            mark_failed(scratch, S, tok, false);
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            // a direct segment's last span writes the header: the invalid one
            if (direct && b + 1 == blocks) write_header<kFb>(args, sg, L, 0, false, false, tok);
            return;
        }
    } else if (table) {
        __syncthreads();  // sh.code ready
    }
    if (kFb && mode == kModeSpecRaw) {
        raw_span(args, s, b, direct, in, table, base_hi, tok, sh);
        return;
    }

    // ---- phase A: split, code, planes; count the span's zero-points
    uint32_t ex[kEncSubTiles][kSteps][2], pl[kEncSubTiles][kSteps], zm[kEncSubTiles][kSteps];
#pragma unroll
    for (int sub = 0; sub < kEncSubTiles; ++sub) {
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            const uint64_t base = span0 + (uint64_t)sub * kTile + 512u * (uint32_t)(wave * kSteps + u) +
                                  8u * (uint32_t)lane;
            const uint32_t *d = in[sub][u].d;
            const uint32_t sm0 = sign_mantissa4(d[0], d[1]);
            const uint32_t sm1 = sign_mantissa4(d[2], d[3]);
            const uint32_t t0 = exponent_high(d[0]), t1 = exponent_high(d[1]);
            const uint32_t t2 = exponent_high(d[2]), t3 = exponent_high(d[3]);
            ex[sub][u][0] = exponents4(t0, t1);
            ex[sub][u][1] = exponents4(t2, t3);
            uint32_t c_lo, c_hi;
            if (!table) {
                c_lo = window_codes4(t0, t1, base_hi);
                c_hi = window_codes4(t2, t3, base_hi);
            } else {
                c_lo = c_hi = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    c_lo |= (uint32_t)sh.code[(ex[sub][u][0] >> (8 * k)) & 0xFFu] << (8 * k);
                    c_hi |= (uint32_t)sh.code[(ex[sub][u][1] >> (8 * k)) & 0xFFu] << (8 * k);
                }
            }
            // values at or past n carry no code bits and are no zero-points
            const uint32_t vm = in[sub][u].vmask;
            pl[sub][u] = codes_to_planes(c_lo, c_hi) & (vm * 0x010101u);
            zm[sub][u] = zero_point_mask(pl[sub][u]) & vm;
            if (vm) store_stream8(out + kHeaderBytes + base, sm0, sm1);
        }
    }
    // ---- direct: the span's counts go out before phase B (waves 0 and 1 hold
    // the first 4096-value group, waves 2 and 3 the second).  Not in a launch
    // with the fallback: there the registers this takes would cost a wave per
    // SIMD, which measured slower.
    uint32_t c0 = 0, c1 = 0;
    DirectState dst{0u, true};
    if (!kFb && direct) {
        static_assert(kEncSubTiles == 1 && kWaves == 4, "a span is one tile, two waves per group");
        uint32_t z = 0;
#pragma unroll
        for (int u = 0; u < kSteps; ++u) z += __builtin_popcount(zm[0][u]);
        z = wave_sum(z);
        if (lane == 0) sh.red[wave] = z;
        __syncthreads();
        c0 = sh.red[0] + sh.red[1];
        c1 = sh.red[2] + sh.red[3];
        dst = direct_publish(args, s, b, c0, c1, tok, sh);
    }

    stamp(1);
    // ---- phase B: ranks, plane regrouping, zero-point staging
    uint32_t running = 0;  // zero-points of the span so far (uniform)
#pragma unroll
    for (int sub = 0; sub < kEncSubTiles; ++sub) {
        const uint64_t tile0 = span0 + (uint64_t)sub * kTile;
#pragma unroll
        for (int u = 0; u < kSteps; ++u) sh.planes[(wave * kSteps + u) * kWave + lane] = pl[sub][u];
        const TileCounts tc = count_tile(zm[sub], lane, wave, sh.wave_total[sub & 1]);
        {
            const uint4 q = reinterpret_cast<const uint4 *>(sh.planes)[tid];
            const uint32_t lo01 = perm(q.y, q.x, 0x05010400u), hi23 = perm(q.w, q.z, 0x05010400u);
            const uint32_t p0 = perm(hi23, lo01, 0x05040100u);
            const uint32_t p1 = perm(hi23, lo01, 0x07060302u);
            const uint32_t p2 = perm(perm(q.w, q.z, 0x0C0C0602u), perm(q.y, q.x, 0x0C0C0602u), 0x05040100u);
            if (tile0 + 32u * (uint32_t)tid < n) {
                const uint64_t off = tile0 / 8 + 4u * (uint32_t)tid;
                store_stream4(out + L.off_p0 + off, p0);
                store_stream4(out + L.off_p1 + off, p1);
                store_stream4(out + L.off_p2 + off, p2);
            }
        }
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            uint32_t m = zm[sub][u], r = running + tc.rank[u];
            while (m) {
                const uint32_t k = __builtin_ctz(m);
                m &= m - 1;
                sh.zp[r++] = (uint8_t)get_byte8(ex[sub][u][0], ex[sub][u][1], k);
            }
        }
        if (tid == 0) {
            sh.group[2 * sub] = tc.first_group;
            sh.group[2 * sub + 1] = tc.tile_total - tc.first_group;
        }
        running += tc.tile_total;
        __syncthreads();  // sh.planes is rewritten by the next sub-tile; sh.zp and sh.group are complete
    }

    const uint32_t T = running;

    // ---- pads the data stores never touch (the last span of the segment)
    if (b == blocks - 1) {
        const uint64_t sm_end = kHeaderBytes + 8 * ((n + 7) / 8);
        for (uint64_t i = sm_end + tid; i < L.off_p0; i += kThreads) out[i] = 0;
        const uint64_t pl_end = 4 * ((n + 31) / 32);
        for (uint64_t i = pl_end + tid; i < L.plane_bytes; i += kThreads) {
            out[L.off_p0 + i] = 0;
            out[L.off_p1 + i] = 0;
            out[L.off_p2 + i] = 0;
        }
        for (uint64_t i = L.off_tab + 4 * (L.groups + 1) + tid; i < L.off_zp; i += kThreads) out[i] = 0;
    }
    if (direct) {
        if (kFb) {
            c0 = sh.group[0];
            c1 = sh.group[1];
            dst = direct_publish(args, s, b, c0, c1, tok, sh);
        }
        direct_finish<kFb>(args, s, b, T, c0, c1, false, dst, tok, sh);
        return;
    }

    // ---- staged: the span's zero-point bytes -> its staging slot
    {
        const __amdgpu_buffer_rsrc_t slot =
            __builtin_amdgcn_make_buffer_rsrc(scratch + S.staging + (uint64_t)b * kEncSpan, 0, kEncSpan, kBufferDword3);
        for (uint32_t i = tid; 16 * i < T; i += kThreads)
            put_staged16(slot, 16 * i, reinterpret_cast<const uint4 *>(sh.zp)[i]);
    }

    // ---- publish: every store of every thread has completed (the staged
    // bytes at the coherence point) before the span word is written
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    stamp(2);
    if (tid == 0)
        put_word(scratch + S.span_words + (uint64_t)kWordBytes * b, tok,
                 sh.group[0] | (sh.group[1] << 16));
}

// Finalize role: block r of a segment places the staged zero-point bytes of
// run r, spans [kRun r, kRun r + count) of the segment.
//   1. It waits for the run's span words, publishes the run word (the run's
//      count) and lands the first batch of staged bytes in LDS.
//   2. It sums the zero-points before the run: the earlier runs of its chunk
//      (kChunkRuns runs) through their run words and the earlier chunks
//      through their chunk words.  The last run of a chunk first sums its
//      chunk's runs and publishes the chunk word, so that no chunk word waits
//      for another one.
//   3. It writes the run's table entries and its zero-point bytes, a landed
//      batch at a time.
//   4. The segment's last run writes the header, unless the segment's
//      failure mark is set.  Its offset needed every earlier chunk word (each
//      published after all run words of its chunk) and its own chunk's run
//      words, so every word that any finalize block of the segment waits for
//      has been published.
template <bool kFb>
__device__ __forceinline__ void finalize_run(const EncArgs &args, uint32_t s, uint32_t r, FinShared &sh) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const EncSeg &sg = args.seg[s];
    const uint64_t n = sg.n;
    const Layout L = layout_for(n);
    const Scratch S = scratch_for(n);
    const uint32_t nb = (uint32_t)enc_blocks(n);
    const uint32_t nr = (uint32_t)ceil_div(nb, kRun);
    const uint32_t first = r * kRun, count = min(kRun, nb - first);
    const bool last_run = r + 1 == nr;
    const uint32_t c = r / kChunkRuns, cfirst = c * kChunkRuns;
    const bool chunk_last = r % kChunkRuns == kChunkRuns - 1 || last_run;
    const uint64_t epoch = read_epoch(args, sg);
    uint8_t *const out = sg.out;
    uint8_t *const scratch = seg_scratch(args, sg);
    uint32_t *const tab = reinterpret_cast<uint32_t *>(out + L.off_tab);

    // ---- 0. the raw fallback: under a raw guess the run only counts (its
    // spans staged nothing)
    bool raw = false, ok = true;
    if (kFb && guesses(sg)) {
        const uint32_t m = await_guess(scratch, S, mix_token(args.tok_lo, args.tok_hi, epoch), sh.red);
        ok = m != kModeAbort;
        raw = m == kModeSpecRaw;
    }

    // ---- 1. the run's span words (threads 0 .. count-1, all in wave 0): the
    // exclusive prefixes of zero-points and of landing units, the run's count.
    // The first round of loads goes out before the token is formed, so that
    // it is in flight with the epoch's load.
    const uint8_t *const sw = scratch + S.span_words + (uint64_t)kWordBytes * first;
    uint64_t w0 = 0, w1 = 0;
    if (ok && (uint32_t)tid < count) load_word(sw + (uint64_t)kWordBytes * tid, w0, w1);
    const Token tok = mix_token(args.tok_lo, args.tok_hi, epoch);
    if (ZC_FAIL_OTHERS && !last_run) {
        mark_failed(scratch, S, tok, false);
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    uint32_t sp[1] = {0};
    // (that round is the wait's first poll: a spin limit of 0 allows none)
    const uint32_t done = kSpinLimit > 0 && (uint32_t)tid < count && word_valid(w0, w1, tok, sp[0]) ? 1u : 0u;
    if (ok) ok = poll_words<1>(sw, count, tok, sp, done);
    ok = __syncthreads_and(ok);
    if (wave == 0) {
        const uint32_t g0 = sp[0] & 0xFFFFu, T = g0 + (sp[0] >> 16), U = (T + 15) / 16;  // 0 past count
        const uint32_t inc = wave_inclusive_scan(T), uinc = wave_inclusive_scan(U);
        if ((uint32_t)lane < count) {
            sh.pre[lane] = inc - T;
            sh.land16[lane] = uinc - U;
            sh.g0[lane] = g0;
        }
        if ((uint32_t)lane + 1 == count) {
            sh.pre[count] = inc;
            sh.land16[count] = uinc;
        }
    }
    __syncthreads();
    const uint32_t A = sh.pre[count];
    stamp(1);
    if (ok && tid == 0) put_word(scratch + S.run_words + (uint64_t)kWordBytes * r, tok, A);

    // ---- staged bytes -> the zero-point array, a batch of spans at a time:
    // spans [j0, j1) whose landing units fit the zone.  The first batch lands
    // while the counts of earlier runs are still awaited (the landing needs only
    // the run's own prefixes; the destination needs those counts).
    uint8_t *const zp = out + L.off_zp;
    const uint8_t *const slots = scratch + S.staging;
    auto batch_end = [&](uint32_t j0, uint32_t u0) {  // largest j1 with land16[j1] - u0 <= kLandBytes / 16
        uint32_t lo = j0 + 1, hi = count;
        while (lo < hi) {
            const uint32_t mid = (lo + hi + 1) / 2;
            if (sh.land16[mid] - u0 <= kLandBytes / 16)
                lo = mid;
            else
                hi = mid - 1;
        }
        return lo;
    };
    // Many spans in a batch: wave w takes spans j0 + w, j0 + w + 4, ...  Fewer
    // spans than waves (spans of many zero-points): the chunks of the spans (64
    // units to land; 128 destination dwords to write) are numbered across the
    // batch and wave w takes every kWaves-th one, so a large span is not left
    // to one wave.
    auto land_batch = [&](uint32_t j0, uint32_t j1, uint32_t u0) {
        if (j1 - j0 < (uint32_t)kWaves) {
            uint32_t g = 0;
            for (uint32_t j = j0; j < j1; ++j) {
                const uint32_t a16 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(sh.land16[j] - u0));
                const uint32_t units =
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)(sh.land16[j + 1] - sh.land16[j]));
                land_span(slots + (uint64_t)(first + j) * kEncSpan, units, sh.land + 16u * a16, lane,
                          ((uint32_t)wave + kWaves - g % kWaves) % kWaves, kWaves);
                g += (units + kWave - 1) / kWave;
            }
            return;
        }
        // Wave w lands a contiguous range of the batch's spans (at most 64), whose
        // landing units are contiguous in LDS: one load instruction covers 64
        // units of several spans; a lane finds the span of its unit among the
        // range's starts (held one per lane).
        const uint32_t per = (j1 - j0 + kWaves - 1) / kWaves;
        for (uint32_t a = j0 + (uint32_t)wave * per; a < min(j1, j0 + ((uint32_t)wave + 1) * per); a += kWave) {
            const uint32_t b = min(min(j1, j0 + ((uint32_t)wave + 1) * per), a + kWave);
            const uint32_t nsp = b - a;
            const uint32_t my_start = (uint32_t)lane < nsp ? sh.land16[a + lane] : 0u;
            const uint32_t ua = (uint32_t)__builtin_amdgcn_readfirstlane((int)sh.land16[a]);
            const uint32_t ub = (uint32_t)__builtin_amdgcn_readfirstlane((int)sh.land16[b]);
            for (uint32_t U0 = ua; U0 < ub; U0 += kWave) {
                const uint32_t U = U0 + (uint32_t)lane;
                uint32_t js = 0, st = ua;  // the last span of the range starting at or before U
                for (uint32_t i = 1; i < nsp; ++i) {
                    const uint32_t si = (uint32_t)__builtin_amdgcn_readlane((int)my_start, (int)i);
                    if (si <= U) {
                        js = i;
                        st = si;
                    }
                }
                if (U < ub)
                    __builtin_amdgcn_global_load_lds(
                        (global_void *)(slots + (uint64_t)(first + a + js) * kEncSpan + 16u * (U - st)),
                        (lds_void *)(sh.land + 16u * (U0 - u0)), 16, 0, kCachePolicySc1);
            }
        }
    };
    uint32_t j0 = 0, j1 = 0, u0 = 0;
    if (ok && !raw) {
        u0 = sh.land16[0];
        j1 = batch_end(0, u0);
        land_batch(0, j1, u0);
    }

    // ---- 2. the zero-points before the run
    uint32_t rsum = 0;  // the chunk's runs before r (the chunk's last run)
    uint32_t P = 0;
    {
        if (chunk_last) {
            uint32_t rp[1] = {0};
            if (ok) ok = poll_words<1>(scratch + S.run_words + (uint64_t)kWordBytes * cfirst, r - cfirst, tok, rp);
            ok = __syncthreads_and(ok);
            rsum = block_sum(rp[0], sh.red);
            if (ok && tid == 0 && r % kChunkRuns == kChunkRuns - 1)
                put_word(scratch + S.chunk_words + (uint64_t)kWordBytes * c, tok, rsum + A);
        }
        if (!raw || last_run) {  // a raw guess: only the header writer needs the offset
            const uint32_t nrun = chunk_last ? 0u : r - cfirst;  // earlier runs of the chunk, then earlier chunks
            uint32_t pp[3] = {0, 0, 0};
            static_assert(kChunkRuns - 1 + ((kMaxElems + kEncSpan - 1) / kEncSpan + kChunkSpans - 1) / kChunkSpans <=
                              3 * kThreads, "one round polls every word");
            if (ok)
                ok = poll_list<3>(
                    nrun + c,
                    [&](uint32_t i) {
                        return i < nrun ? scratch + S.run_words + (uint64_t)kWordBytes * (cfirst + i)
                                        : scratch + S.chunk_words + (uint64_t)kWordBytes * (i - nrun);
                    },
                    tok, pp);
            ok = __syncthreads_and(ok);
            P = rsum + block_sum(pp[0] + pp[1] + pp[2], sh.red);
        }
    }
    if (ZC_FAIL_OTHERS && !last_run) ok = false;
    mark_failed(scratch, S, tok, ok);
    // the header writer: the failure mark, read once its own waits have passed
    // (in flight while it writes the run's bytes)
    uint64_t fa = 0, fb = 0;
    if (last_run) load_word(scratch + S.failed, fa, fb);

    stamp(2);
    // ---- 3. table entries and zero-point bytes
    if (ok && !raw) {
        if ((uint32_t)tid < count) {
            const uint64_t gi = (uint64_t)(first + tid) * kEncGroups;
            const uint32_t p0 = P + sh.pre[tid];
            if (gi < L.groups) tab[gi] = p0;
            if (gi + 1 < L.groups) tab[gi + 1] = p0 + sh.g0[tid];
        }
        const uint32_t Pu = (uint32_t)__builtin_amdgcn_readfirstlane((int)P);
        for (;;) {
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();  // the batch has landed
            const bool split = j1 - j0 < (uint32_t)kWaves;
            if (split) {
                uint32_t g = 0;
                for (uint32_t j = j0; j < j1; ++j) {
                    const uint32_t p = (uint32_t)__builtin_amdgcn_readfirstlane((int)sh.pre[j]);
                    const uint32_t T = (uint32_t)__builtin_amdgcn_readfirstlane((int)sh.pre[j + 1]) - p;
                    const uint64_t dst = (uint64_t)Pu + p;
                    write_span(zp, dst, sh.land + 16u * (sh.land16[j] - u0), T, lane,
                               ((uint32_t)wave + kWaves - g % kWaves) % kWaves, kWaves);
                    g += (span_dwords(dst, T) + 2 * kWave - 1) / (2 * kWave);
                }
            } else {
                // four of the wave's spans at a time, 16 lanes each
                const uint32_t grp = (uint32_t)lane >> 4, gl = (uint32_t)lane & 15u;
                for (uint32_t jq = j0 + (uint32_t)wave; jq < j1; jq += 4u * kWaves) {
                    const uint32_t j = jq + grp * kWaves;
                    if (j < j1) {
                        const uint32_t p = sh.pre[j], T = sh.pre[j + 1] - p;
                        write_span_group(zp, (uint64_t)Pu + p, sh.land + 16u * (sh.land16[j] - u0), T, gl);
                    }
                }
            }
            j0 = j1;
            if (j0 >= count) break;
            __syncthreads();  // the landing zone is reused
            u0 = sh.land16[j0];
            j1 = batch_end(j0, u0);
            land_batch(j0, j1, u0);
        }
    }
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no landing left in flight (a given-up call)

    // ---- 4. the header of a segment without direct spans
    if (last_run) {
        uint32_t f;
        if (word_valid(fa, fb, tok, f)) ok = false;
        ok = __syncthreads_and(ok);
        write_header<kFb>(args, sg, L, (uint64_t)P + A, ok, kFb && raw, tok);
    }
}

// The role of block blockIdx.x: its piece's kind and segment, and its first
// unit (span of an encoder piece, run of a finalize piece).
struct BlockRole {
    uint32_t kind, seg, unit, p;
};
__device__ __forceinline__ BlockRole block_role(const EncArgs &args, uint32_t mult) {
    const uint32_t flat = blockIdx.x;
    const uint32_t p = find_piece(args, flat);
    const uint32_t w = args.piece[p];
    return BlockRole{(w >> 24) & 3u, w >> 26, args.first[p] + (flat - (w & kBlockMask)) * mult, p};
}

// Sampler role (the raw fallback's first launch): the guess for segment s,
// published in its decision word.  The sampler blocks open the grid, so the
// guesses are out before the segments' own blocks look for them.
__device__ __forceinline__ void sample_segment(const EncArgs &args, uint32_t s, EncShared &sh) {
    const EncSeg &sg = args.seg[s];
    if (!guesses(sg)) return;
    const Token tok = launch_token(args, sg);
    const bool table = (sg.flags & kSegTable) != 0;
    if (table) {
        uint32_t c = 0;
#pragma unroll
        for (int k = 0; k < 7; ++k) c = (sg.exps[k] == (uint32_t)threadIdx.x) ? (uint32_t)(k + 1) : c;
        sh.code[threadIdx.x] = (uint8_t)c;
        __syncthreads();
    }
    const uint32_t wbase = (uint32_t)sg.exps[0] - 1u;  // window mode only (exps[0] >= 1)
    const uint32_t base_hi = (wbase << 8) | (wbase << 24);
    const Layout L = layout_for(sg.n);
    const uint32_t d = sample_guess(sg, L, table, base_hi, sh.code, sh.red);
    if (threadIdx.x == 0) put_word(seg_scratch(args, sg) + scratch_for(sg.n).decision, tok, d);
}

// One block of a compress launch, one unit.  kFb: the launch has segments
// under the raw fallback (the first launch of such a call).
template <bool kFb>
__device__ __forceinline__ void compress_block(const EncArgs &args, CompressShared &sh) {
    const BlockRole r = block_role(args, 1);
    stamp(0);
    stamp_role(r.kind, r.seg, r.unit);
    if (kFb && r.kind == kPieceSample) {
        sample_segment(args, r.unit, sh.e);
    } else if (r.kind == kPieceFinalize) {
        // A finalize block's waves issue ahead of the encoder waves sharing its
        // CU: finalize work must keep up with the encoding it follows.
        __builtin_amdgcn_s_setprio(2);
        finalize_run<kFb>(args, r.seg, r.unit, sh.f);
    } else {
        encode_span<kFb>(args, r.seg, r.unit, r.kind == kPieceDirect, sh.e);
    }
    stamp(3);
}

// Launches without the fallback.  Eight waves per SIMD: the register budget
// for that (at most 64 VGPRs, and at most 80 SGPRs as the code object counts
// them: measured on gfx950, 80 still gives eight 256-thread blocks per CU and
// 81 gives seven) is requested explicitly, so that a few SGPRs more in the
// code do not silently cost a block per CU; the compiler then keeps surplus
// scalars in VGPR lanes.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void compress_kernel(
    EncArgs args) {
    __shared__ CompressShared sh;
    compress_block<false>(args, sh);
}

// The first launch of a call with segments under the raw fallback.  Seven
// waves per SIMD (at most 72 VGPRs, 94 SGPRs), asked for explicitly: eight
// would spill registers to scratch, which measured slower than seven.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(7, 8))) void compress_fallback_kernel(
    EncArgs args) {
    __shared__ CompressShared sh;
    compress_block<true>(args, sh);
}

// The second launch of a call with segments under the raw fallback, over
// those segments only, args.mult units per block (most blocks only read their
// segment's status word, and a launch pays per block) on a staged grid.  A
// segment that came out raw after a coded pass gets its payload copied; a
// wrong raw guess gets a plain coded pass (the outcome is known to be coded),
// unit by unit in each block's order.
__global__ __launch_bounds__(kThreads) void compress_second_kernel(EncArgs args) {
    __shared__ CompressShared sh;
    const BlockRole r = block_role(args, args.mult);
    const EncSeg &sg = args.seg[r.seg];
    const uint32_t u1 = (uint32_t)min((uint64_t)r.unit + args.mult,
                                      piece_end(r.kind, args.first[r.p], enc_blocks(sg.n), args.chunk));
    const uint32_t mode = second_pass_mode(args, sg);
    if (mode == kModeSkip) return;
    if (mode == kModeCopyRaw) {
        if (r.kind != kPieceFinalize)
            for (uint32_t u = r.unit; u < u1; ++u) copy_span_raw(sg.in, sg.out, (uint64_t)u * kEncSpan, sg.n);
        return;
    }
    // one loop per role: a loop holding both roles needs twice the registers
    if (r.kind == kPieceFinalize) {
        __builtin_amdgcn_s_setprio(2);
        for (uint32_t u = r.unit; u < u1; ++u) {
            if (u != r.unit) __syncthreads();  // the previous unit is done with the LDS
            finalize_run<false>(args, r.seg, u, sh.f);
        }
    } else {
        for (uint32_t u = r.unit; u < u1; ++u) {
            if (u != r.unit) __syncthreads();
            encode_span<false>(args, r.seg, u, false, sh.e);
        }
    }
}

}  // namespace zc

// ===========================================================================
// C ABI
// ===========================================================================

using namespace zc;

// Per-call tokens: splitmix64 (Steele, Lea, Flood, "Fast splittable
// pseudorandom number generators", 2014) of a process-wide counter whose
// start is drawn once from the OS entropy source and the clock.  splitmix64 is
// a bijection, so no two calls of a process share a token.
static uint64_t splitmix64(uint64_t x) {
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

static uint64_t next_token() {
    static std::atomic<uint64_t> counter{[] {
        std::random_device rd;
        const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
        return ((uint64_t)rd() << 32) ^ (uint64_t)rd() ^ splitmix64(t);
    }()};
    return splitmix64(counter.fetch_add(1, std::memory_order_relaxed));
}

// The raw fallback's second launch gives each block this many units: most of
// its blocks only read a status word, and a launch pays per block.
constexpr uint32_t kSecondPassMult = 16;

// One compress launch over a.seg[0 .. a.k), its grid laid out here; second:
// the fallback's second launch (a staged grid, several units per block).
static zc_status launch_compress(EncArgs &a, hipStream_t st, bool second) {
    const uint32_t mult = second ? kSecondPassMult : 1u;
    uint64_t ns[ZC_MAX_BATCH];
    for (uint32_t i = 0; i < a.k; ++i) ns[i] = a.seg[i].n;
    GridPlan grid;
    bool fb = false;
    for (uint32_t i = 0; i < a.k; ++i) fb |= (a.seg[i].flags & kSegRawOk) != 0;
    if (!plan_grid(ns, a.k, grid, mult, second, fb && !second)) return ZC_ERR_INVALID_ARG;
    std::memcpy(a.piece, grid.piece, sizeof(a.piece));
    std::memcpy(a.first, grid.first, sizeof(a.first));
    a.pieces = grid.pieces;
    a.mult = mult;
    a.chunk = (uint32_t)grid.chunk;
    // every block follows the blocks it waits for (zc_grid.h): workgroups are
    // dispatched in index order, so each of those has been dispatched first
    const dim3 blocks(grid.piece[grid.pieces]);
    if (second)
        hipLaunchKernelGGL(compress_second_kernel, blocks, dim3(kThreads), 0, st, a);
    else if (fb)
        hipLaunchKernelGGL(compress_fallback_kernel, blocks, dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(compress_kernel, blocks, dim3(kThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? ZC_OK : ZC_ERR_HIP;
}

// Compress with the scratch in `ws` (ws_bytes, 256-byte aligned; segment i's
// scratch at the sum of zc_compress_workspace_bytes over the segments before
// it), or, ws null, behind each stream in its output buffer.
static zc_status compress_impl(const zc_enc_seg *segs, uint32_t k, void *ws, uint64_t ws_bytes, void *stream) {
    if (!segs || k == 0 || k > ZC_MAX_BATCH) return ZC_ERR_INVALID_ARG;
    if (ws && ((uintptr_t)ws & 255u)) return ZC_ERR_MISALIGNED;
    EncArgs a;
    std::memset(&a, 0, sizeof(a));
    a.ws = static_cast<uint8_t *>(ws);
    uint64_t ws_used = 0;
    for (uint32_t i = 0; i < k; ++i) {
        const zc_enc_seg &g = segs[i];
        if (!g.out || g.n > kMaxElems || (g.n && !g.in) || !zc_plan_is_valid(&g.plan)) return ZC_ERR_INVALID_ARG;
        if (((uintptr_t)g.in & 15u) || ((uintptr_t)g.out & 127u) || ((uintptr_t)g.out_bytes & 7u))
            return ZC_ERR_MISALIGNED;
        const uint64_t seg_ws = zc_compress_workspace_bytes(g.n);
        if (g.out_capacity < zc_max_compressed_bytes(g.n) + (ws ? 0 : seg_ws)) return ZC_ERR_CAPACITY;
        EncSeg &e = a.seg[i];
        if (ws) {
            if (ws_used / 256 > 0xFFFFFFFFull) return ZC_ERR_INVALID_ARG;
            e.ws_off = (uint32_t)(ws_used / 256);
            ws_used += seg_ws;
        }
        e.in = static_cast<const uint16_t *>(g.in);
        e.out = static_cast<uint8_t *>(g.out);
        e.out_bytes = reinterpret_cast<unsigned long long *>(g.out_bytes);
        e.n = (uint32_t)g.n;
        std::memcpy(e.exps, g.plan.exps, 7);
        // exps = w+1 .. w+7 with w >= 0: codes by saturating arithmetic; any
        // other ascending set: codes from a 256-byte LDS table
        const bool window = g.plan.exps[0] >= 1 && g.plan.exps[6] - g.plan.exps[0] == 6;
        e.flags = (uint8_t)((window ? 0 : kSegTable) | ((g.plan.flags & ZC_PLAN_RAW_FALLBACK) ? kSegRawOk : 0));
    }
    if (ws && ws_used > ws_bytes) return ZC_ERR_CAPACITY;
    a.k = k;
    const uint64_t tok = next_token();
    a.tok_lo = (uint32_t)tok;
    a.tok_hi = (uint32_t)(tok >> 32);
    a.advance = 1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    zc_status rc = launch_compress(a, st, false);
    if (rc != ZC_OK) return rc;
    // The raw fallback's second launch, over the flagged segments only: it
    // completes what the first left (the payload of a stream that came out
    // raw, or the coded stream of a wrong raw guess).  The two launches are
    // ordered on the stream, so it sees every word and byte of the first.
    EncArgs b;
    std::memset(&b, 0, sizeof(b));
    for (uint32_t i = 0; i < k; ++i)
        if (a.seg[i].flags & kSegRawOk) b.seg[b.k++] = a.seg[i];
    if (!b.k) return ZC_OK;
    const uint64_t tok2 = next_token();
    b.tok_lo = (uint32_t)tok2;
    b.tok_hi = (uint32_t)(tok2 >> 32);
    b.prev_lo = a.tok_lo;
    b.prev_hi = a.tok_hi;
    b.ws = a.ws;
    return launch_compress(b, st, true);
}

#ifdef ZC_TIMELINE
// The instrumented build's timeline: clear it before a launch, read it after
// (both synchronous; 0 on success).
extern "C" int zc_timeline_clear() {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(zc::zc_timeline)) != hipSuccess) return 1;
    if (hipMemset(p, 0, sizeof(zc::zc_timeline)) != hipSuccess) return 1;
    return hipDeviceSynchronize() == hipSuccess ? 0 : 1;
}
extern "C" int zc_timeline_read(void *dst, uint64_t bytes) {
    if (bytes > sizeof(zc::zc_timeline)) bytes = sizeof(zc::zc_timeline);
    return hipMemcpyFromSymbol(dst, HIP_SYMBOL(zc::zc_timeline), bytes, 0, hipMemcpyDeviceToHost) == hipSuccess ? 0
                                                                                                       : 1;
}
#endif

extern "C" zc_status zc_compress_batch(const zc_enc_seg *segs, uint32_t k, void *stream) {
    return compress_impl(segs, k, nullptr, 0, stream);
}

extern "C" zc_status zc_compress_batch_ws(const zc_enc_seg *segs, uint32_t k, void *d_workspace,
                                          uint64_t workspace_bytes, void *stream) {
    if (!d_workspace) return ZC_ERR_INVALID_ARG;
    return compress_impl(segs, k, d_workspace, workspace_bytes, stream);
}

extern "C" zc_status zc_compress(const void *d_in, uint64_t n, const zc_plan *plan, void *d_out,
                                 uint64_t out_capacity, uint64_t *d_out_bytes, void *stream) {
    if (!plan) return ZC_ERR_INVALID_ARG;
    zc_enc_seg s;
    s.in = d_in;
    s.n = n;
    s.plan = *plan;
    s.out = d_out;
    s.out_capacity = out_capacity;
    s.out_bytes = d_out_bytes;
    return zc_compress_batch(&s, 1, stream);
}

extern "C" zc_status zc_compress_ws(const void *d_in, uint64_t n, const zc_plan *plan, void *d_out,
                                    uint64_t out_capacity, uint64_t *d_out_bytes, void *d_workspace,
                                    uint64_t workspace_bytes, void *stream) {
    if (!plan) return ZC_ERR_INVALID_ARG;
    zc_enc_seg s;
    s.in = d_in;
    s.n = n;
    s.plan = *plan;
    s.out = d_out;
    s.out_capacity = out_capacity;
    s.out_bytes = d_out_bytes;
    return zc_compress_batch_ws(&s, 1, d_workspace, workspace_bytes, stream);
}
