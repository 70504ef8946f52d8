// Local reduction of the reduce-scatter path (section 2.D of the ZipCCL
// explainer pages: a reduce-scatter run as a zipped all-to-all followed by a
// local reduction) and its C ABI, MI355X / gfx950: k streams of the same n
// BF16 values are decoded and summed in float32, in stream order, onto the
// local share, and the sums rounded to BF16 once.
#include <hip/hip_runtime.h>

#include <cstring>

#include "zc.h"
#include "zc_device.h"
#include "zc_format.h"
#include "zc_lane.h"

namespace zc {

// Local reduction of the reduce-scatter path: k streams of the same n values.
struct RedStream {
    const uint8_t *in;
    uint64_t in_bytes;
};

struct RedArgs {
    uint32_t k;
    uint32_t n;
    const uint16_t *local;  // nullable
    uint16_t *out;
    int32_t *status;        // nullable
    RedStream s[ZC_MAX_BATCH];
};

// ---------------------------------------------------------------------------
// local reduction of the reduce-scatter path (section 2.D): decode k streams
// of the same n values and add them
// ---------------------------------------------------------------------------

// BF16 value pair of a dword -> two floats (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Nearest BF16 to a float, ties to even (the bias 0x7FFF plus the lowest kept
// bit carries into the kept half exactly when the dropped half is above one
// half, or equal to it with an odd kept half); a NaN gives 0x7FC0.
__device__ __forceinline__ uint32_t float_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    return (f != f) ? 0x7FC0u : ((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Work split.  A 4096-value tile (one zero-point group) is decoded by two
// waves, one per 2048-value half, each lane owning 32 consecutive values; a
// block holds two tiles.  The waves do not wait for each other while they
// work: each keeps its lanes' sign+mantissa and plane words in registers (the
// next stream's in flight while the current one is decoded) and stages its
// own zero-point slice in LDS.  Half 0's zero-points start at the group's
// table entry and half 1's end at the next group's, so neither needs the
// other's count.  At the end the two halves of a tile compare, stream by
// stream, where the first one's zero-points end and the second one's begin: a
// table that disagrees with the planes sets the status.
constexpr uint32_t kRedTile = 4096;
static_assert(kRedTile == kGroup, "a tile is one zero-point group");
constexpr uint32_t kRedHalf = kRedTile / 2;
static_assert(kRedHalf / kWave == 32, "a lane's zero-point flags fill one dword");
constexpr uint32_t kRedTilesPerBlock = kWaves / 2;
// Zero-point bytes a wave stages per stream (a quarter of its tile's values).
// A half with more zero-points than that reads them from memory one by one.
constexpr uint32_t kRedSliceCap = 1024;
// the staged bytes from a dword-aligned start (up to 3 bytes of lead-in), and
// the gather's 3-dword reads at the last zero-point
constexpr uint32_t kRedSliceWords = 260;
static_assert(kRedSliceWords >= (kRedSliceCap + 3) / 4 + 3, "room for the gather's reads");

// Per-stream facts of a checked header, kept in LDS: E (two words), the code
// table (two words).  Bit 31 of E's high word marks a raw stream.
struct RedHdr {
    uint32_t e_lo, e_hi, tbl_lo, tbl_hi;
};

struct RedShared {
    uint32_t slice[kWaves][2][kRedSliceWords];  // before the first stream: every header's 32 words
    uint32_t edge[kWaves][ZC_MAX_BATCH];        // per stream: where half 0's zero-points end / half 1's begin
    RedHdr hdr[ZC_MAX_BATCH];
    uint2 sel[256];
};
static_assert(sizeof(RedShared::slice) >= 4u * 32u * ZC_MAX_BATCH, "room for every header");

// Every stream's header at once: the 32 words of each go to LDS with one
// vector load per thread and word (all in flight together), then thread s
// checks stream s.  Returns the block-wide verdict; hdr[s] receives stream s's
// facts.  `words` (k * 32 words) may alias memory that is not yet in use.
__device__ __forceinline__ bool red_check_headers(const RedArgs &args, uint64_t n, const Layout &L, uint32_t *words,
                                                  RedHdr *hdr) {
    const uint32_t k = args.k, tid = threadIdx.x;
    for (uint32_t i = tid; i < 32u * k; i += kThreads)
        words[i] = *reinterpret_cast<const uint32_t *>(args.s[i / 32].in + 4u * (i % 32));
    __syncthreads();
    bool ok = true;
    if (tid < k) {
        const uint32_t *w = words + 32u * tid;
        uint32_t pad = 0;
        for (int i = 12; i < 32; ++i) pad |= w[i];
        const uint64_t E = w[8] | ((uint64_t)w[9] << 32);
        const uint64_t total = w[10] | ((uint64_t)w[11] << 32);
        const uint32_t h6 = w[6], h7 = w[7];
        const uint32_t mode = h7 >> 24;
        const bool raw = mode == kModeRaw;
        const bool sized = ((mode == kModeCoded) & (total == L.off_zp + E)) | (raw & (total == kHeaderBytes + 2 * n));
        ok = (w[0] == kMagic) & (w[1] == ((uint32_t)kVersion | (kHeaderBytes << 16))) & (w[2] == (uint32_t)n) &
             (w[3] == (uint32_t)(n >> 32)) & (w[4] == kGroup) & (w[5] == (uint32_t)L.groups) & sized & (E <= n) &
             (total <= args.s[tid].in_bytes) & (pad == 0u);
        const uint32_t e[7] = {h6 & 0xFFu, (h6 >> 8) & 0xFFu, (h6 >> 16) & 0xFFu, h6 >> 24,
                               h7 & 0xFFu, (h7 >> 8) & 0xFFu, (h7 >> 16) & 0xFFu};
        for (int j = 1; j < 7; ++j) ok = ok & (e[j] > e[j - 1]);
        RedHdr r;
        r.e_lo = (uint32_t)E;
        r.e_hi = (uint32_t)(E >> 32) | (raw ? 0x80000000u : 0u);
        r.tbl_lo = h6 << 8;
        r.tbl_hi = (h6 >> 24) | (h7 << 8);
        hdr[tid] = r;
    }
    return __syncthreads_and(ok);
}

// Uniform per-stream facts of a checked header.  E <= n < 2^32.
struct RedMeta {
    const uint8_t *in;
    uint64_t in_bytes;
    uint32_t E;
    uint32_t tbl_lo, tbl_hi;  // exponent of code c in byte c of {tbl_hi:tbl_lo} (byte 0 unused)
    bool raw;
};

__device__ __forceinline__ RedMeta red_meta(const RedArgs &args, uint32_t s, const RedHdr *hdr) {
    RedMeta m;
    m.in = args.s[s].in;
    m.in_bytes = args.s[s].in_bytes;
    const uint4 h = *reinterpret_cast<const uint4 *>(hdr + s);
    m.E = (uint32_t)__builtin_amdgcn_readfirstlane((int)h.x);
    m.raw = ((uint32_t)__builtin_amdgcn_readfirstlane((int)h.y) >> 31) != 0u;
    m.tbl_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)h.z);
    m.tbl_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)h.w);
    return m;
}

// s_waitcnt immediate (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): vmcnt(0), the others unconstrained.
constexpr int kWaitVm0 = 0x0F70;

// Wait for every load of the wave, direct-to-LDS ones included, as a compiler
// barrier as well (inline assembly with a memory clobber): no LDS read moves
// above it.  Used where the reads of LDS that such loads wrote do not depend
// on any later load.
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Lanes of one wave exchanging data through LDS: the wave's LDS accesses
// complete in order, so waiting for its own is enough; the memory clobber
// keeps the compiler from moving accesses across (per lane, the addresses
// written and read look unrelated).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Direct-to-LDS dword load, written as inline assembly so that the compiler
// adds no waits of its own for it; the kernel waits with an explicit count.
// The LDS address is the wave-uniform base in M0 plus 4 bytes per lane.
__device__ __forceinline__ uint32_t lds_base(const void *lds) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)lds);
}
__device__ __forceinline__ void lds_load4(const void *src, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off nt" ::"s"(m0), "v"(src)
                 : "memory", "m0");
}

// The lane's values: [v0, v0 + nv) inside the stream, nv = 0..32.
struct RedLane {
    uint64_t v0;
    uint32_t nv;
    uint32_t vmask;   // bit i: value v0 + i exists
    uint32_t sm_off;  // byte offsets of its sign+mantissa bytes and plane words (0 past the end: always readable)
    uint32_t pl_off;
};

// The lane's sign+mantissa bytes (32) and plane words (one per plane).
struct RedData {
    uint4 sm0, sm1;
    uint32_t p0, p1, p2;
};

__device__ __forceinline__ void red_load(RedData &d, const RedMeta &m, const Layout &L, const RedLane &ln) {
    const uint8_t *sm = m.in + kHeaderBytes;
    const uint8_t *pl = m.in + L.off_p0;
    d.sm0 = load_stream16(sm + ln.sm_off);
    d.sm1 = load_stream16(sm + ln.sm_off + 16u);
    d.p0 = load_stream4(pl + ln.pl_off);
    d.p1 = load_stream4(pl + L.plane_bytes + ln.pl_off);
    d.p2 = load_stream4(pl + 2 * L.plane_bytes + ln.pl_off);
}

// Zero-points [lo, lo + len) of a stream into buf: whole dwords direct to
// LDS (from the dword holding zero-point lo); a partial last dword is read
// whole when the buffer holds all of it, else byte by byte.
__device__ __forceinline__ void red_stage_range(const RedMeta &m, const Layout &L, uint32_t lo, uint32_t len,
                                                uint32_t *buf, int lane) {
    const uint64_t A0 = L.off_zp + lo, A1 = A0 + len;
    const uint64_t a0 = A0 & ~uint64_t(3);
    const uint64_t a1 = (A1 + 3 <= m.in_bytes) ? ((A1 + 3) & ~uint64_t(3)) : (A1 & ~uint64_t(3));
    const uint32_t ndw = (uint32_t)((a1 - a0) / 4);
    for (uint32_t i0 = 0; i0 < ndw; i0 += kWave)
        if (i0 + (uint32_t)lane < ndw) lds_load4(m.in + a0 + 4u * (i0 + (uint32_t)lane), lds_base(buf + i0));
    if (A1 > a1 && lane == 0) {  // a partial dword at the very end of the buffer
        uint32_t w = 0;
        for (uint32_t i = 0; i < (uint32_t)(A1 - a1); ++i) w |= (uint32_t)m.in[a1 + i] << (8 * i);
        buf[ndw] = w;
    }
}

// Table entries of tile t, checked and clamped to the stream (a mismatch sets
// bad), and the zero-points [lo, lo + len) the wave stages in buf: the first
// ones of the group for half 0, the last ones for half 1, at most
// kRedSliceCap.
__device__ __forceinline__ void red_stage(const RedMeta &m, const Layout &L, uint32_t t, bool last, uint32_t half,
                                          uint32_t &z0, uint32_t &z1, uint32_t &lo, uint32_t &len, uint32_t *buf,
                                          int lane, bool &bad) {
    const_u32 *tab = (const_u32 *)(m.in + L.off_tab);
    z0 = tab[t];
    z1 = tab[t + 1];  // t + 1 <= groups: the table's last entry at most
    if ((t == 0 && z0 != 0) || (last && z1 != m.E)) bad = true;
    if (z0 > m.E) { bad = true; z0 = m.E; }
    if (z1 < z0 || z1 > m.E) { bad = true; z1 = z1 < z0 ? z0 : m.E; }
    if (z1 - z0 > kRedTile) { bad = true; z1 = z0 + kRedTile; }
    len = min(z1 - z0, kRedSliceCap);
    lo = half ? z1 - len : z0;
    red_stage_range(m, L, lo, len, buf, lane);
}

// Plane bytes of the lane's 8-value unit u: [plane 0, plane 1, plane 2, 0].
__device__ __forceinline__ uint32_t red_planes(const RedData &d, uint32_t u) {
    const uint32_t w01 = perm(d.p1, d.p0, u | ((4u + u) << 8) | 0x0C0C0000u);
    return perm(d.p2, w01, 0x0100u | ((4u + u) << 16) | 0x0C000000u);
}

// Adds 8 values (sign+mantissa dwords sm_lo / sm_hi, exponent bytes e_lo /
// e_hi) to acc8.  The float of a BF16 value has the value's high byte (sign,
// exponent >> 1) on top and its low byte (exponent & 1, mantissa) below it:
// one byte select per value.
__device__ __forceinline__ void red_add8(float *acc8, uint32_t sm_lo, uint32_t sm_hi, uint32_t e_lo, uint32_t e_hi) {
    const uint32_t h0 = bfi(0x80808080u, sm_lo, e_lo >> 1), l0 = bfi(0x7F7F7F7Fu, sm_lo, e_lo << 7);
    const uint32_t h1 = bfi(0x80808080u, sm_hi, e_hi >> 1), l1 = bfi(0x7F7F7F7Fu, sm_hi, e_hi << 7);
#pragma unroll
    for (uint32_t j = 0; j < 4; ++j) {
        const uint32_t sel = 0x0C0Cu | (j << 16) | ((4u + j) << 24);
        acc8[j] += __uint_as_float(perm(h0, l0, sel));
        acc8[4 + j] += __uint_as_float(perm(h1, l1, sel));
    }
}

// The wave's zero-point flags (bit i: value v0 + i of the lane) and their
// exclusive prefix count over the lanes; returns the wave's count.
__device__ __forceinline__ uint32_t red_flags(const RedData &d, const RedLane &ln, uint32_t &z32, uint32_t &excl) {
    z32 = ~(d.p0 | d.p1 | d.p2) & ln.vmask;
    const uint32_t cnt = (uint32_t)__builtin_popcount(z32);
    const uint32_t incl = wave_inclusive_scan(cnt);
    excl = incl - cnt;
    return (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
}

// Where a raw stream's (or the local share's) values are read: the tile's
// values wv (uniform; the tile's first value always exists), the lane's byte
// offset from there, whether all 2048 values of the wave exist (uniform).
// When not, the lane reads value by value from tail_off (its own offset, or 0
// for a lane past the end), at most value tail_last (nv - 1, or 0) from there.
struct RedRaw {
    const uint8_t *wv;
    uint32_t lane_off;
    bool full;
    uint32_t tail_off, tail_last;
};

// The 8 values of unit u of a raw stream as 4 BF16 pairs (missing values
// repeat an existing one; their sums are never stored).
__device__ __forceinline__ void red_raw_unit(const RedRaw &rw, uint32_t u, uint32_t (&w)[4]) {
    if (rw.full) {
        const uint4 v = load_stream16(rw.wv + (rw.lane_off + 16u * u));
        w[0] = v.x;
        w[1] = v.y;
        w[2] = v.z;
        w[3] = v.w;
    } else {
        // (an opaque copy: offsets computed from it are not hoisted out of the
        // stream loop, where they would hold 32 registers)
        uint32_t lastv = rw.tail_last, loff = rw.tail_off;
        asm volatile("" : "+v"(lastv), "+v"(loff));
#pragma unroll
        for (uint32_t j = 0; j < 4; ++j) {
            const uint32_t i = 8u * u + 2u * j;
            const uint32_t lo = *reinterpret_cast<const uint16_t *>(rw.wv + (loff + 2u * min(i, lastv)));
            const uint32_t hi = *reinterpret_cast<const uint16_t *>(rw.wv + (loff + 2u * min(i + 1u, lastv)));
            w[j] = lo | (hi << 16);
        }
    }
}

// Decodes the lane's 32 values of a stream and adds them to acc.  Coded: the
// lane's first zero-point is byte r0 of buf and each 8-value unit's are
// contiguous there.  Raw: the values are read as they are and split like the
// encoder splits them (sign+mantissa bytes, exponent bytes), so that every
// stream's values enter the sums through the same instructions.
__device__ __forceinline__ void red_decode(const RedMeta &m, const RedData &d, uint32_t z32, uint32_t r0,
                                           const uint32_t *buf, const uint2 *sel, const RedRaw &rw,
                                           float (&acc)[32]) {
    const uint32_t smw[8] = {d.sm0.x, d.sm0.y, d.sm0.z, d.sm0.w, d.sm1.x, d.sm1.y, d.sm1.z, d.sm1.w};
#pragma unroll
    for (uint32_t u = 0; u < 4; ++u) {
        uint32_t sm_lo, sm_hi, e_lo, e_hi;
        if (m.raw) {
            uint32_t w[4];
            red_raw_unit(rw, u, w);
            sm_lo = sign_mantissa4(w[0], w[1]);
            sm_hi = sign_mantissa4(w[2], w[3]);
            e_lo = exponents4(exponent_high(w[0]), exponent_high(w[1]));
            e_hi = exponents4(exponent_high(w[2]), exponent_high(w[3]));
        } else {
            uint32_t c_lo, c_hi;
            planes_to_codes(red_planes(d, u), c_lo, c_hi);
            e_lo = perm(m.tbl_hi, m.tbl_lo, c_lo);
            e_hi = perm(m.tbl_hi, m.tbl_lo, c_hi);
            const uint32_t r = u ? r0 + (uint32_t)__builtin_popcount(z32 & ((1u << (8u * u)) - 1u)) : r0;
            put_zero_points(e_lo, e_hi, (z32 >> (8u * u)) & 0xFFu, r, buf, sel);
            sm_lo = smw[2u * u];
            sm_hi = smw[2u * u + 1u];
        }
        red_add8(acc + 8u * u, sm_lo, sm_hi, e_lo, e_hi);
        __builtin_amdgcn_sched_barrier(0);  // one unit's registers live at a time
    }
}

// A block checks every stream's header first (a bad header anywhere leaves the
// whole output untouched), then each wave decodes its half-tile of every
// stream in order.  The float32 sums start from the local value, or from -0.0
// (-0.0 + x is x for every x, so the first stream enters exactly).
__global__ __launch_bounds__(kThreads) void reduce_kernel(RedArgs args) {
    __shared__ RedShared sh;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: tile, half and addresses in SGPRs
    const uint64_t n = args.n;
    const Layout L = layout_for(n);
    const uint32_t k = args.k;
    const uint32_t half = (uint32_t)wave & 1u;
    const uint32_t t = blockIdx.x * kRedTilesPerBlock + (uint32_t)wave / 2;
    const bool active = t < L.groups;
    const bool last = t + 1 == L.groups;

    zp_selectors(sh.sel);  // visible after the barriers of the header check
    if (!red_check_headers(args, n, L, &sh.slice[0][0][0], sh.hdr)) {
        if (tid == 0 && args.status) *args.status = ZC_ERR_CORRUPT;
        return;
    }

    RedLane ln;
    ln.v0 = (uint64_t)t * kRedTile + kRedHalf * half + 32u * (uint32_t)lane;
    ln.nv = ln.v0 < n ? (uint32_t)min(n - ln.v0, (uint64_t)32) : 0u;
    ln.vmask = ln.nv == 32 ? ~0u : (1u << ln.nv) - 1u;
    ln.sm_off = ln.nv ? (uint32_t)ln.v0 : 0u;
    ln.pl_off = ln.nv ? (uint32_t)(ln.v0 / 8) : 0u;

    // where the lane reads BF16 arrays (the local share, raw streams)
    const uint64_t tile0 = (uint64_t)t * kRedTile;
    RedRaw rw;
    rw.lane_off = 2u * (kRedHalf * half + 32u * (uint32_t)lane);
    rw.full = tile0 + kRedHalf * (half + 1u) <= n;
    rw.tail_off = ln.nv ? rw.lane_off : 0u;
    rw.tail_last = ln.nv ? ln.nv - 1u : 0u;

    // A wave whose 2048 values all exist moves its local share in and its
    // result out through its slice buffers (free at both times), in two
    // rounds of 1024 values: each global access instruction then covers 1 KiB
    // of consecutive bytes, where lanes of 32 consecutive values would touch
    // every cache line in part (measured: a quarter of the kernel's time).
    uint8_t *const xpose = reinterpret_cast<uint8_t *>(sh.slice[wave][0]);
    static_assert(sizeof(RedShared::slice[0]) >= 2048, "a round of 1024 values fits a wave's slice buffers");
    const uint64_t half0 = tile0 + kRedHalf * half;  // the wave's first value

    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = -0.0f;
    if (args.local && active) {
        if (rw.full) {
#pragma unroll
            for (uint32_t r = 0; r < 2; ++r) {
                const uint8_t *src = reinterpret_cast<const uint8_t *>(args.local + half0 + 1024u * r);
                const uint4 a = load_stream16(src + 16u * (uint32_t)lane);
                const uint4 b = load_stream16(src + 1024u + 16u * (uint32_t)lane);
                *reinterpret_cast<uint4 *>(xpose + 16u * (uint32_t)lane) = a;
                *reinterpret_cast<uint4 *>(xpose + 1024u + 16u * (uint32_t)lane) = b;
                wave_lds_sync();
                if ((uint32_t)lane / 32u == r) {
                    const uint8_t *mine = xpose + 64u * ((uint32_t)lane % 32u);
#pragma unroll
                    for (uint32_t q = 0; q < 4; ++q) {
                        const uint4 v = *reinterpret_cast<const uint4 *>(mine + 16u * q);
                        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (uint32_t j = 0; j < 4; ++j) {
                            acc[8 * q + 2 * j] = bf16_lo(w[j]);
                            acc[8 * q + 2 * j + 1] = bf16_hi(w[j]);
                        }
                    }
                }
                wave_lds_sync();  // (the next round rewrites the buffer: reads first)
            }
        } else {
            rw.wv = reinterpret_cast<const uint8_t *>(args.local + tile0);
#pragma unroll
            for (uint32_t u = 0; u < 4; ++u) {
                uint32_t w[4];
                red_raw_unit(rw, u, w);
#pragma unroll
                for (uint32_t j = 0; j < 4; ++j) {
                    acc[8 * u + 2 * j] = bf16_lo(w[j]);
                    acc[8 * u + 2 * j + 1] = bf16_hi(w[j]);
                }
            }
        }
    }

    bool bad = false;
    if (active && k) {
        RedMeta cur = red_meta(args, 0, sh.hdr);
        RedData dc, dn;
        uint32_t z0 = 0, z1 = 0, lo = 0, len = 0;
        if (!cur.raw) {
            red_stage(cur, L, t, last, half, z0, z1, lo, len, sh.slice[wave][0], lane, bad);
            red_load(dc, cur, L, ln);
        }
        for (uint32_t s = 0; s < k; ++s) {
            // Stream s's words and slice have landed.  (This wait orders no LDS
            // read for the compiler; it does not need to: the slice's reads
            // take their addresses from stream s's plane words, which the
            // compiler waits for, and the slice was issued before them.)
            __builtin_amdgcn_s_waitcnt(kWaitVm0);
            RedMeta nxt = cur;
            uint32_t nz0 = 0, nz1 = 0, nlo = 0, nlen = 0;
            const bool staged = s + 1 < k && !(nxt = red_meta(args, s + 1, sh.hdr)).raw;
            if (staged) {  // the next stream's slice and words go out now
                red_stage(nxt, L, t, last, half, nz0, nz1, nlo, nlen, sh.slice[wave][(s + 1) & 1u], lane, bad);
                red_load(dn, nxt, L, ln);
            }
            uint32_t edge = 0, z32 = 0, r0 = 0, x = s & 1u;
            bool heavy = false;
            rw.wv = cur.in + kHeaderBytes + 2 * tile0;
            if (!cur.raw) {
                uint32_t excl;
                const uint32_t c = red_flags(dc, ln, z32, excl);
                edge = half ? z1 - c : z0 + c;
                // half 0's zero-points open the staged slice, half 1's close it
                r0 = (lo & 3u) + (half ? len - c : 0u) + excl;
                heavy = c > len;
                if (heavy) {
                    // More zero-points than staged (or than the table allows): the
                    // half's own ones, at most 2048 bytes, go to both slice buffers
                    // (back to back); the next stream's slice is staged again after.
                    const uint32_t a = half ? (c <= z1 ? z1 - c : 0u) : z0;
                    wait_loads();
                    red_stage_range(cur, L, a, min(c, cur.E - a), sh.slice[wave][0], lane);
                    wait_loads();
                    r0 = (a & 3u) + excl;
                    x = 0;
                }
            }
            red_decode(cur, dc, z32, r0, sh.slice[wave][x], sh.sel, rw, acc);
            if (heavy && staged) {
                red_stage_range(nxt, L, nlo, nlen, sh.slice[wave][(s + 1) & 1u], lane);
                wait_loads();  // (issued after the next stream's plane words: not covered by waiting for them)
            }
            if (lane == 0) sh.edge[wave][s] = edge;
            cur = nxt;
            dc = dn;
            z0 = nz0;
            z1 = nz1;
            lo = nlo;
            len = nlen;
        }
    }
    __syncthreads();  // the edges of both halves
    if (active && half == 0)
        for (uint32_t s = (uint32_t)lane; s < k; s += kWave)
            if (sh.edge[wave][s] != sh.edge[wave + 1][s]) bad = true;

    if (active) {
        uint32_t o[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) o[i] = float_to_bf16(acc[2 * i]) | (float_to_bf16(acc[2 * i + 1]) << 16);
        if (rw.full) {
#pragma unroll
            for (uint32_t r = 0; r < 2; ++r) {
                if ((uint32_t)lane / 32u == r) {
                    uint8_t *mine = xpose + 64u * ((uint32_t)lane % 32u);
#pragma unroll
                    for (uint32_t q = 0; q < 4; ++q)
                        *reinterpret_cast<uint4 *>(mine + 16u * q) =
                            make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
                }
                wave_lds_sync();
                uint8_t *dst = reinterpret_cast<uint8_t *>(args.out + half0 + 1024u * r);
                const uint4 a = *reinterpret_cast<const uint4 *>(xpose + 16u * (uint32_t)lane);
                const uint4 b = *reinterpret_cast<const uint4 *>(xpose + 1024u + 16u * (uint32_t)lane);
                store_stream16(dst + 16u * (uint32_t)lane, a.x, a.y, a.z, a.w);
                store_stream16(dst + 1024u + 16u * (uint32_t)lane, b.x, b.y, b.z, b.w);
                wave_lds_sync();  // (the next round rewrites the buffer: reads first)
            }
        } else if (ln.nv) {
            uint16_t *dst = args.out + ln.v0;
#pragma unroll
            for (uint32_t i = 0; i < 32; ++i)
                if (i < ln.nv) dst[i] = (uint16_t)(o[i / 2] >> (16 * (i % 2)));
        }
    }
    if (bad && args.status) atomicMax(args.status, (int32_t)ZC_ERR_CORRUPT);
}

}  // namespace zc

// ===========================================================================
// C ABI
// ===========================================================================

using namespace zc;

extern "C" zc_status zc_decompress_reduce(const void *const *d_streams, const uint64_t *in_bytes, uint32_t k,
                                          uint64_t n, const void *d_local, void *d_out, int32_t *d_status,
                                          void *stream) {
    if (k > ZC_MAX_BATCH || (k && (!d_streams || !in_bytes)) || (k == 0 && !d_local) || n > kMaxElems ||
        (n && !d_out))
        return ZC_ERR_INVALID_ARG;
    if (((uintptr_t)d_local & 15u) || ((uintptr_t)d_out & 15u) || ((uintptr_t)d_status & 3u))
        return ZC_ERR_MISALIGNED;
    RedArgs a;
    std::memset(&a, 0, sizeof(a));
    const Layout L = layout_for(n);
    for (uint32_t i = 0; i < k; ++i) {
        if (!d_streams[i]) return ZC_ERR_INVALID_ARG;
        if ((uintptr_t)d_streams[i] & 127u) return ZC_ERR_MISALIGNED;
        // no stream of n values is shorter than both forms
        if (in_bytes[i] < L.off_zp && in_bytes[i] < kHeaderBytes + 2 * n) return ZC_ERR_CORRUPT;
        a.s[i].in = static_cast<const uint8_t *>(d_streams[i]);
        a.s[i].in_bytes = in_bytes[i];
    }
    a.k = k;
    a.n = (uint32_t)n;
    a.local = static_cast<const uint16_t *>(d_local);
    a.out = static_cast<uint16_t *>(d_out);
    a.status = d_status;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (d_status) {
        ZeroArgs z;
        std::memset(&z, 0, sizeof(z));
        z.count = 1;
        z.r[0].ptr = reinterpret_cast<uint32_t *>(d_status);
        z.r[0].words = 1;
        const zc_status rc = launch_zero(z, st);
        if (rc != ZC_OK) return rc;
    }
    // n = 0 still runs one block: every header is checked, nothing is written
    const uint64_t tiles = (n + kRedTile - 1) / kRedTile;
    const uint64_t blocks = tiles ? (tiles + kRedTilesPerBlock - 1) / kRedTilesPerBlock : 1;
    hipLaunchKernelGGL(reduce_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? ZC_OK : ZC_ERR_HIP;
}
