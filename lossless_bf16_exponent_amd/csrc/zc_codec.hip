// HIP kernels and C ABI of the BF16 exponent-coding codec for MI355X (gfx950).
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
//   * a 256-thread block codes one 8192-element tile; a lane loads 8 values
//     with one 128-bit load per step, so every wave-wide load or store is a
//     contiguous 1 KiB (input), 512 B (sign+mantissa) or 64 B (plane) run;
//   * codes and bit planes come from dword-wide byte shuffles (zc_lane.h), and
//     the per-lane plane bytes are regrouped through LDS into whole dwords per
//     plane before they are stored;
//   * zero-point bytes are placed by an exclusive scan: lane (packed 16-bit
//     wave scan) -> wave (LDS) -> sub-tile -> block span (single-pass
//     decoupled look-back over 64-bit flag+count words, one per block of
//     kEncSubTiles tiles, so its latency is paid once per 32768 values and
//     overlaps the next blocks' streaming);
//   * the decoder needs no scan across tiles: the table of zero-point counts
//     per 4096-element group gives every tile its slice of the zero-point
//     array, which is staged in LDS and gathered by rank.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>

#include "zc.h"
#include "zc_format.h"
#include "zc_lane.h"

namespace zc {

// ---------------------------------------------------------------------------
// kernel arguments (passed by value; at most ZC_MAX_BATCH segments)
// ---------------------------------------------------------------------------

struct EncSeg {
    const uint16_t *in;
    uint8_t *out;
    unsigned long long *out_bytes;
    uint32_t n;
    uint32_t tile_begin;  // first flat block of this segment
    uint8_t exps[7];
    uint8_t mode;  // kModeWindow or kModeTable
};
static_assert(sizeof(EncSeg) == 40, "compact kernel arguments");

struct EncArgs {
    uint32_t k;
    uint32_t total_blocks;
    EncSeg seg[ZC_MAX_BATCH];
};

struct DecSeg {
    const uint8_t *in;
    uint16_t *out;
    int32_t *status;
    uint64_t in_bytes;
    uint32_t n;
    uint32_t tile_begin;
};
static_assert(sizeof(DecSeg) == 40, "compact kernel arguments");

struct DecArgs {
    uint32_t k;
    uint32_t total_tiles;
    DecSeg seg[ZC_MAX_BATCH];
};

struct ZeroRegion {
    uint32_t *ptr;
    uint64_t words;
};

struct ZeroArgs {
    uint32_t count;
    ZeroRegion r[ZC_MAX_BATCH];
};

constexpr uint8_t kModeWindow = 0;  // exps = w+1 .. w+7 with w >= 0: codes by saturating arithmetic
constexpr uint8_t kModeTable = 1;   // any other ascending set: codes from a 256-byte LDS table

// look-back word: flag in the high 32 bits, zero-point count in the low 32
constexpr uint64_t kFlagAggregate = 1ull << 32;
constexpr uint64_t kFlagPrefix = 2ull << 32;
constexpr uint32_t kSpinLimit = 1u << 20;

// ---------------------------------------------------------------------------
// streaming memory access: every codec byte is read once and written once,
// so loads and stores carry the non-temporal hint (measured on MI355X: a
// 128-bit copy moves 13 % more bytes per second with it)
// ---------------------------------------------------------------------------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_stream16(const void *p) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint2 load_stream8(const void *p) {
    const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    return make_uint2(t.x, t.y);
}
__device__ __forceinline__ uint32_t load_stream4(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
}
__device__ __forceinline__ void store_stream16(void *p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u32x4 t = {a, b, c, d};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ void store_stream8(void *p, uint32_t a, uint32_t b) {
    const u32x2 t = {a, b};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x2 *>(p));
}
__device__ __forceinline__ void store_stream4(void *p, uint32_t a) {
    __builtin_nontemporal_store(a, reinterpret_cast<uint32_t *>(p));
}

// ---------------------------------------------------------------------------
// wave helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        uint32_t o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

__device__ __forceinline__ uint32_t find_segment_enc(const EncArgs &a, uint32_t flat) {
    uint32_t s = 0;
    for (uint32_t i = 1; i < a.k; ++i)
        if (a.seg[i].tile_begin <= flat) s = i;
    return s;
}

__device__ __forceinline__ uint32_t find_segment_dec(const DecArgs &a, uint32_t flat) {
    uint32_t s = 0;
    for (uint32_t i = 1; i < a.k; ++i)
        if (a.seg[i].tile_begin <= flat) s = i;
    return s;
}

// Zero-point counts of the four steps of a lane -> tile-local ranks of the
// lane's first zero-point value in each step, plus the wave and tile totals.
// Order inside a tile: wave-major, then step, then lane, then value.
struct TileCounts {
    uint32_t rank[kSteps];
    uint32_t tile_total;
    uint32_t first_group;  // zero-points among the tile's first 4096 values (waves 0, 1)
};

__device__ __forceinline__ TileCounts count_tile(const uint32_t (&zmask)[kSteps], int lane, int wave,
                                                 uint32_t *s_wave_total) {
    static_assert(kSteps == 4, "two packed 16-bit scans cover four steps");
    uint32_t c[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) c[u] = __builtin_popcount(zmask[u]);
    const uint32_t a = c[0] | (c[1] << 16), b = c[2] | (c[3] << 16);
    const uint32_t ai = wave_inclusive_scan(a, lane), bi = wave_inclusive_scan(b, lane);
    const uint32_t at = __shfl(ai, kWave - 1, kWave), bt = __shfl(bi, kWave - 1, kWave);
    const uint32_t ae = ai - a, be = bi - b;
    const uint32_t tot[kSteps] = {at & 0xFFFFu, at >> 16, bt & 0xFFFFu, bt >> 16};
    const uint32_t ex[kSteps] = {ae & 0xFFFFu, ae >> 16, be & 0xFFFFu, be >> 16};
    if (lane == 0) s_wave_total[wave] = tot[0] + tot[1] + tot[2] + tot[3];
    __syncthreads();
    uint32_t wave_off = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const uint32_t v = s_wave_total[w];
        wave_off += (w < wave) ? v : 0u;
        total += v;
    }
    TileCounts r;
    uint32_t run = wave_off;
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
        r.rank[u] = run + ex[u];
        run += tot[u];
    }
    r.tile_total = total;
    r.first_group = s_wave_total[0] + s_wave_total[1];
    static_assert(kGroup == 2 * kWave * 8 * kSteps, "a group is the span of two waves");
    return r;
}

// ---------------------------------------------------------------------------
// small fill kernel: look-back scratch before an encode, status words before a decode
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void zero_kernel(ZeroArgs a) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint32_t i = 0; i < a.count; ++i) {
        uint32_t *p = a.r[i].ptr;
        const uint64_t words = a.r[i].words;
        for (uint64_t w = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; w < words; w += stride) p[w] = 0;
    }
}

// ---------------------------------------------------------------------------
// encoder
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

// A block codes kEncSubTiles consecutive 8192-value sub-tiles (its span).
// All loads of the span are issued up front.  Phase A turns every step into
// sign+mantissa bytes (stored at once), exponent bytes and plane bytes, and
// counts the span's zero-point values; the count is published right away so
// that later blocks' look-backs never wait for this block's stores.  Phase B
// then ranks, regroups and stages, while wave 0's look-back is in flight.
// Blocks are ordered by blockIdx: workgroups are dispatched in index order,
// so a block only ever waits for blocks that are already running or done; the
// wait is bounded regardless.
__global__ __launch_bounds__(kThreads) void encode_kernel(EncArgs args) {
    __shared__ uint32_t s_planes[kTile / 8];     // per 8-value group: plane bytes 0, 1, 2
    __shared__ uint8_t s_zp[kEncSpan];           // the span's zero-point bytes, in order
    __shared__ uint8_t s_code[256];              // table mode: exponent -> code
    __shared__ uint32_t s_wave_total[2][kWaves];
    __shared__ uint32_t s_group[kEncGroups];     // zero-points per 4096-value group of the span
    __shared__ uint32_t s_prefix;

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const uint32_t flat = blockIdx.x;
    const uint32_t s = find_segment_enc(args, flat);
    const EncSeg &sg = args.seg[s];
    const uint32_t b = flat - sg.tile_begin;  // block (span) index inside the segment
    const uint64_t n = sg.n;
    const Layout L = layout_for(n);
    const uint64_t blocks = enc_blocks(n);
    const uint8_t mode = sg.mode;
    const uint64_t span0 = (uint64_t)b * kEncSpan;
    uint8_t *const out = sg.out;
    uint8_t *const scratch = out + L.off_scratch;
    unsigned long long *const state = reinterpret_cast<unsigned long long *>(scratch + kScratchCtrl);

    if (mode == kModeTable) {
        uint32_t c = 0;
#pragma unroll
        for (int k = 0; k < 7; ++k) c = (sg.exps[k] == (uint32_t)tid) ? (uint32_t)(k + 1) : c;
        s_code[tid] = (uint8_t)c;
    }
    const uint32_t wbase = (uint32_t)sg.exps[0] - 1u;  // window mode only (exps[0] >= 1)
    const uint32_t base_hi = (wbase << 8) | (wbase << 24);

    // ---- every load of the span in flight at once
    Step in[kEncSubTiles][kSteps];
#pragma unroll
    for (int sub = 0; sub < kEncSubTiles; ++sub)
#pragma unroll
        for (int u = 0; u < kSteps; ++u)
            in[sub][u] = load_step(sg.in, span0 + (uint64_t)sub * kTile + 512u * (uint32_t)(wave * kSteps + u) +
                                              8u * (uint32_t)lane, n);
    if (mode == kModeTable) __syncthreads();  // s_code ready

    // ---- phase A: split, code, planes; count the span's zero-points
    uint32_t ex[kEncSubTiles][kSteps][2], pl[kEncSubTiles][kSteps], zm[kEncSubTiles][kSteps];
    uint32_t lane_zeros = 0;
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
            if (mode == kModeWindow) {
                c_lo = window_codes4(t0, t1, base_hi);
                c_hi = window_codes4(t2, t3, base_hi);
            } else {
                c_lo = c_hi = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    c_lo |= (uint32_t)s_code[(ex[sub][u][0] >> (8 * k)) & 0xFFu] << (8 * k);
                    c_hi |= (uint32_t)s_code[(ex[sub][u][1] >> (8 * k)) & 0xFFu] << (8 * k);
                }
            }
            // values at or past n carry no code bits and are no zero-points
            const uint32_t vm = in[sub][u].vmask;
            pl[sub][u] = codes_to_planes(c_lo, c_hi) & (vm * 0x010101u);
            zm[sub][u] = zero_point_mask(pl[sub][u]) & vm;
            lane_zeros += __builtin_popcount(zm[sub][u]);
            if (vm) store_stream8(out + kHeaderBytes + base, sm0, sm1);
        }
    }
    {
        const uint32_t wz = wave_sum(lane_zeros);
        if (lane == 0) s_wave_total[1][wave] = wz;
    }
    __syncthreads();
    const uint32_t T = s_wave_total[1][0] + s_wave_total[1][1] + s_wave_total[1][2] + s_wave_total[1][3];

    // ---- publish the span's count, and start looking back
    unsigned long long lb_value = kFlagPrefix;
    int64_t lb_idx = (int64_t)b - 1;
    if (wave == 0) {
        if (lane == 0)
            __hip_atomic_store(&state[b], (b == 0 ? kFlagPrefix : kFlagAggregate) | T, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        const int64_t j = lb_idx - lane;
        if (b > 0 && j >= 0) lb_value = __hip_atomic_load(&state[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- phase B: ranks, plane regrouping, zero-point staging
    uint32_t running = 0;  // zero-points of the span so far (uniform)
#pragma unroll
    for (int sub = 0; sub < kEncSubTiles; ++sub) {
        const uint64_t tile0 = span0 + (uint64_t)sub * kTile;
#pragma unroll
        for (int u = 0; u < kSteps; ++u) s_planes[(wave * kSteps + u) * kWave + lane] = pl[sub][u];
        const TileCounts tc = count_tile(zm[sub], lane, wave, s_wave_total[sub & 1]);
        {
            const uint4 q = reinterpret_cast<const uint4 *>(s_planes)[tid];
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
                s_zp[r++] = (uint8_t)get_byte8(ex[sub][u][0], ex[sub][u][1], k);
            }
        }
        if (tid == 0) {
            s_group[2 * sub] = tc.first_group;
            s_group[2 * sub + 1] = tc.tile_total - tc.first_group;
        }
        running += tc.tile_total;
        __syncthreads();  // s_planes is rewritten by the next sub-tile
    }

    // ---- span prefix: finish the decoupled look-back (wave 0)
    if (wave == 0) {
        uint32_t prefix = 0;
        if (b > 0) {
            unsigned long long v = lb_value;
            uint32_t spins = 0;
            for (;;) {
                const uint32_t flag = (uint32_t)(v >> 32);
                const unsigned long long pmask = __ballot(flag == 2u);
                const unsigned long long zmask_lb = __ballot(flag == 0u);
                const unsigned long long upto = pmask ? (pmask & (0ull - pmask)) * 2ull - 1ull : ~0ull;
                if (zmask_lb & upto) {
                    if (++spins > kSpinLimit) {
                        if (lane == 0) atomicOr(reinterpret_cast<uint32_t *>(scratch + 8), 1u);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                } else {
                    prefix += wave_sum(((upto >> lane) & 1ull) ? (uint32_t)v : 0u);
                    if (pmask) break;
                    lb_idx -= kWave;
                }
                const int64_t j = lb_idx - lane;
                v = j >= 0 ? __hip_atomic_load(&state[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : kFlagPrefix;
            }
            if (lane == 0)
                __hip_atomic_store(&state[b], kFlagPrefix | (uint64_t)(prefix + T), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        if (lane == 0) s_prefix = prefix;
    }
    __syncthreads();
    const uint32_t prefix = s_prefix;
    const bool last = (b == blocks - 1);

    // ---- zero-point table entries of the span's groups (the last span also
    // writes the closing entry, E)
    if (tid <= kEncGroups) {
        const uint64_t g = (uint64_t)b * kEncGroups + tid;
        if (g <= L.groups && (tid < kEncGroups || last)) {
            uint32_t before = prefix;
            for (int j = 0; j < tid; ++j) before += s_group[j];
            reinterpret_cast<uint32_t *>(out + L.off_tab)[g] = before;
        }
    }

    // ---- zero-point bytes (a prefix past n can only follow a look-back
    // timeout, which has already marked the stream invalid; never write past
    // the zero-point section then)
    if ((uint64_t)prefix + T <= n) {
        uint8_t *zp = out + L.off_zp + prefix;
        for (uint32_t i = tid; i < T; i += kThreads) zp[i] = s_zp[i];
    }

    // ---- the last span writes the header, the pads and the size
    if (last) {
        const uint64_t E = (uint64_t)prefix + T;
        const uint64_t total = L.off_zp + E;
        const uint32_t err = __hip_atomic_load(reinterpret_cast<uint32_t *>(scratch + 8), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        if (tid < 32) {
            uint32_t w = 0;
            switch (tid) {
                case 0: w = err ? 0u : kMagic; break;
                case 1: w = (uint32_t)kVersion | (kHeaderBytes << 16); break;
                case 2: w = (uint32_t)n; break;
                case 3: w = (uint32_t)(n >> 32); break;
                case 4: w = kGroup; break;
                case 5: w = (uint32_t)L.groups; break;
                case 6: w = sg.exps[0] | (sg.exps[1] << 8) | (sg.exps[2] << 16) | ((uint32_t)sg.exps[3] << 24); break;
                case 7: w = sg.exps[4] | (sg.exps[5] << 8) | (sg.exps[6] << 16); break;
                case 8: w = (uint32_t)E; break;
                case 9: w = (uint32_t)(E >> 32); break;
                case 10: w = (uint32_t)total; break;
                case 11: w = (uint32_t)(total >> 32); break;
                default: break;
            }
            reinterpret_cast<uint32_t *>(out)[tid] = w;
        }
        // pads the data stores above never touch
        const uint64_t sm_end = kHeaderBytes + 8 * ((n + 7) / 8);
        for (uint64_t i = sm_end + tid; i < L.off_p0; i += kThreads) out[i] = 0;
        const uint64_t pl_end = 4 * ((n + 31) / 32);
        for (uint64_t i = pl_end + tid; i < L.plane_bytes; i += kThreads) {
            out[L.off_p0 + i] = 0;
            out[L.off_p1 + i] = 0;
            out[L.off_p2 + i] = 0;
        }
        for (uint64_t i = L.off_tab + 4 * (L.groups + 1) + tid; i < L.off_zp; i += kThreads) out[i] = 0;
        if (tid == 0 && sg.out_bytes) *sg.out_bytes = total;
    }
}

// ---------------------------------------------------------------------------
// decoder
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t ld_u32(const uint8_t *p) { return *reinterpret_cast<const uint32_t *>(p); }

__global__ __launch_bounds__(kThreads) void decode_kernel(DecArgs args) {
    __shared__ uint32_t s_planes[kTile / 8];
    __shared__ uint8_t s_zp[kTile];
    __shared__ uint32_t s_wave_total[kWaves];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const uint32_t flat = blockIdx.x;
    const uint32_t s = find_segment_dec(args, flat);
    const DecSeg &sg = args.seg[s];
    const uint32_t t = flat - sg.tile_begin;
    const uint64_t n = sg.n;
    const Layout L = layout_for(n);
    const uint8_t *const in = sg.in;

    // ---- header: every block checks it, so a bad header stops all of them
    const uint32_t h6 = ld_u32(in + 24), h7 = ld_u32(in + 28);
    const uint64_t E = ld_u32(in + 32) | ((uint64_t)ld_u32(in + 36) << 32);
    const uint64_t total = ld_u32(in + 40) | ((uint64_t)ld_u32(in + 44) << 32);
    bool ok = ld_u32(in) == kMagic && ld_u32(in + 4) == ((uint32_t)kVersion | (kHeaderBytes << 16)) &&
              ld_u32(in + 8) == (uint32_t)n && ld_u32(in + 12) == (uint32_t)(n >> 32) && ld_u32(in + 16) == kGroup &&
              ld_u32(in + 20) == (uint32_t)L.groups && (h7 >> 24) == 0u && E <= n && total == L.off_zp + E &&
              total <= sg.in_bytes;
    {
        const uint32_t e[7] = {h6 & 0xFFu, (h6 >> 8) & 0xFFu, (h6 >> 16) & 0xFFu, h6 >> 24,
                               h7 & 0xFFu, (h7 >> 8) & 0xFFu, (h7 >> 16) & 0xFFu};
#pragma unroll
        for (int k = 1; k < 7; ++k) ok = ok && e[k] > e[k - 1];
#pragma unroll
        for (int w = 12; w < 32; ++w) ok = ok && ld_u32(in + 4 * w) == 0u;
    }
    if (!ok) {
        if (tid == 0 && sg.status) *sg.status = ZC_ERR_CORRUPT;
        return;
    }
    // code -> exponent table for v_perm: byte 0 (code 000) is a placeholder
    const uint32_t tbl_lo = h6 << 8, tbl_hi = (h6 >> 24) | (h7 << 8);

    // ---- this tile's slice of the zero-point array
    const uint32_t *tab = reinterpret_cast<const uint32_t *>(in + L.off_tab);
    const uint64_t g = 2ull * t;
    uint32_t z0 = tab[g];
    uint32_t z1 = tab[g + 1 <= L.groups ? g + 1 : L.groups];
    uint32_t z2 = tab[g + 2 <= L.groups ? g + 2 : L.groups];
    const bool last = (t == L.tiles - 1);
    bool bad = !(z0 <= z1 && z1 <= z2 && z2 <= E) || (t == 0 && z0 != 0) || (last && z2 != E) || z2 - z0 > kTile;
    if (bad) {  // keep every read inside the stream and inside s_zp
        z0 = z0 < E ? z0 : (uint32_t)E;
        z1 = z1 < z0 ? z0 : (z1 > E ? (uint32_t)E : z1);
        z2 = z2 < z1 ? z1 : (z2 > E ? (uint32_t)E : z2);
        if (z2 - z0 > kTile) z2 = z0 + kTile;
    }
    const uint32_t zcount = z2 - z0;
    for (uint32_t i = tid; i < zcount; i += kThreads) s_zp[i] = in[L.off_zp + z0 + i];

    // ---- planes: one dword of each plane per thread, interleaved into LDS
    {
        uint32_t p0 = 0, p1 = 0, p2 = 0;
        const uint64_t tile0 = (uint64_t)t * kTile;
        if (tile0 + 32u * (uint32_t)tid < n) {
            const uint64_t off = tile0 / 8 + 4u * (uint32_t)tid;
            p0 = load_stream4(in + L.off_p0 + off);
            p1 = load_stream4(in + L.off_p1 + off);
            p2 = load_stream4(in + L.off_p2 + off);
        }
        const uint32_t lo = perm(p1, p0, 0x05010400u), hi = perm(p1, p0, 0x07030602u);
        uint4 q;
        q.x = perm(p2, lo, 0x0C040100u);
        q.y = perm(p2, lo, 0x0C050302u);
        q.z = perm(p2, hi, 0x0C060100u);
        q.w = perm(p2, hi, 0x0C070302u);
        reinterpret_cast<uint4 *>(s_planes)[tid] = q;
    }

    // ---- sign+mantissa bytes
    const uint64_t tile0 = (uint64_t)t * kTile;
    uint32_t sm[kSteps][2], vmask[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
        const uint64_t base = tile0 + 512u * (uint32_t)(wave * kSteps + u) + 8u * (uint32_t)lane;
        sm[u][0] = sm[u][1] = 0;
        vmask[u] = 0;
        if (base < n) {
            const uint2 v = load_stream8(in + kHeaderBytes + base);
            sm[u][0] = v.x;
            sm[u][1] = v.y;
            vmask[u] = base + 8 <= n ? 0xFFu : (1u << (uint32_t)(n - base)) - 1u;
        }
    }
    __syncthreads();  // s_planes, s_zp

    uint32_t e[kSteps][2], zmask[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
        const uint32_t planes = s_planes[(wave * kSteps + u) * kWave + lane] & 0x00FFFFFFu;
        uint32_t c_lo, c_hi;
        planes_to_codes(planes, c_lo, c_hi);
        e[u][0] = perm(tbl_hi, tbl_lo, c_lo);
        e[u][1] = perm(tbl_hi, tbl_lo, c_hi);
        zmask[u] = zero_point_mask(planes) & vmask[u];
    }
    const TileCounts tc = count_tile(zmask, lane, wave, s_wave_total);
    if (tc.tile_total != zcount || (uint64_t)z0 + tc.first_group != z1) bad = true;
    if (bad && tid == 0 && sg.status) atomicMax(sg.status, (int32_t)ZC_ERR_CORRUPT);

#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
        uint32_t m = zmask[u], r = tc.rank[u];
        while (m) {
            const uint32_t k = __builtin_ctz(m);
            m &= m - 1;
            const uint32_t b = r < zcount ? s_zp[r] : 0u;
            ++r;
            put_byte8(e[u][0], e[u][1], k, b);
        }
        const uint64_t base = tile0 + 512u * (uint32_t)(wave * kSteps + u) + 8u * (uint32_t)lane;
        uint32_t o0, o1, o2, o3;
        rebuild4(sm[u][0], e[u][0], o0, o1);
        rebuild4(sm[u][1], e[u][1], o2, o3);
        if (vmask[u] == 0xFFu) {
            store_stream16(sg.out + base, o0, o1, o2, o3);
        } else if (vmask[u]) {
            const uint32_t w4[4] = {o0, o1, o2, o3};
            for (uint32_t i = 0; base + i < n; ++i) sg.out[base + i] = (uint16_t)(w4[i / 2] >> (16 * (i % 2)));
        }
    }
}

}  // namespace zc

// ===========================================================================
// C ABI
// ===========================================================================

using namespace zc;

static bool plan_ok(const zc_plan &p) {
    if (p.reserved != 0) return false;
    for (int k = 1; k < 7; ++k)
        if (p.exps[k] <= p.exps[k - 1]) return false;
    return true;
}

static zc_status launch_zero(ZeroArgs &z, hipStream_t st) {
    uint64_t words = 0;
    for (uint32_t i = 0; i < z.count; ++i) words += z.r[i].words;
    if (!words) return ZC_OK;
    uint64_t blocks = (words + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(zero_kernel, dim3((uint32_t)blocks), dim3(256), 0, st, z);
    return hipGetLastError() == hipSuccess ? ZC_OK : ZC_ERR_HIP;
}

extern "C" uint64_t zc_max_compressed_bytes(uint64_t n) {
    if (n > kMaxElems) return 0;
    return layout_for(n).off_scratch + scratch_bytes(n);
}

extern "C" zc_status zc_compress_batch(const zc_enc_seg *segs, uint32_t k, void *stream) {
    if (!segs || k == 0 || k > ZC_MAX_BATCH) return ZC_ERR_INVALID_ARG;
    EncArgs a;
    std::memset(&a, 0, sizeof(a));
    ZeroArgs z;
    std::memset(&z, 0, sizeof(z));
    uint64_t tiles = 0;
    for (uint32_t i = 0; i < k; ++i) {
        const zc_enc_seg &g = segs[i];
        if (!g.out || g.n > kMaxElems || (g.n && !g.in) || !plan_ok(g.plan)) return ZC_ERR_INVALID_ARG;
        if (((uintptr_t)g.in & 15u) || ((uintptr_t)g.out & 127u) || ((uintptr_t)g.out_bytes & 7u))
            return ZC_ERR_MISALIGNED;
        if (g.out_capacity < zc_max_compressed_bytes(g.n)) return ZC_ERR_CAPACITY;
        const Layout L = layout_for(g.n);
        EncSeg &e = a.seg[i];
        e.in = static_cast<const uint16_t *>(g.in);
        e.out = static_cast<uint8_t *>(g.out);
        e.out_bytes = reinterpret_cast<unsigned long long *>(g.out_bytes);
        e.n = (uint32_t)g.n;
        e.tile_begin = (uint32_t)tiles;
        std::memcpy(e.exps, g.plan.exps, 7);
        e.mode = (g.plan.exps[0] >= 1 && g.plan.exps[6] - g.plan.exps[0] == 6) ? kModeWindow : kModeTable;
        const uint64_t blocks = enc_blocks(g.n);
        tiles += blocks;
        if (tiles > 0xFFFFFFFFull) return ZC_ERR_INVALID_ARG;
        z.r[i].ptr = reinterpret_cast<uint32_t *>(e.out + L.off_scratch);
        z.r[i].words = (kScratchCtrl + 8 * blocks) / 4;
    }
    a.k = k;
    a.total_blocks = (uint32_t)tiles;
    z.count = k;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    zc_status rc = launch_zero(z, st);
    if (rc != ZC_OK) return rc;
    hipLaunchKernelGGL(encode_kernel, dim3(a.total_blocks), dim3(kThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? ZC_OK : ZC_ERR_HIP;
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

extern "C" zc_status zc_decompress_batch(const zc_dec_seg *segs, uint32_t k, void *stream) {
    if (!segs || k == 0 || k > ZC_MAX_BATCH) return ZC_ERR_INVALID_ARG;
    DecArgs a;
    std::memset(&a, 0, sizeof(a));
    ZeroArgs z;
    std::memset(&z, 0, sizeof(z));
    uint64_t tiles = 0;
    for (uint32_t i = 0; i < k; ++i) {
        const zc_dec_seg &g = segs[i];
        if (!g.in || g.n > kMaxElems || (g.n && !g.out)) return ZC_ERR_INVALID_ARG;
        if (((uintptr_t)g.in & 127u) || ((uintptr_t)g.out & 15u) || ((uintptr_t)g.status & 3u))
            return ZC_ERR_MISALIGNED;
        const Layout L = layout_for(g.n);
        if (g.in_bytes < L.off_zp) return ZC_ERR_CORRUPT;  // no stream of n values is this short
        DecSeg &d = a.seg[i];
        d.in = static_cast<const uint8_t *>(g.in);
        d.out = static_cast<uint16_t *>(g.out);
        d.status = g.status;
        d.in_bytes = g.in_bytes;
        d.n = (uint32_t)g.n;
        d.tile_begin = (uint32_t)tiles;
        tiles += L.tiles;
        if (tiles > 0xFFFFFFFFull) return ZC_ERR_INVALID_ARG;
        if (g.status) {
            z.r[z.count].ptr = reinterpret_cast<uint32_t *>(g.status);
            z.r[z.count].words = 1;
            ++z.count;
        }
    }
    a.k = k;
    a.total_tiles = (uint32_t)tiles;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    zc_status rc = launch_zero(z, st);
    if (rc != ZC_OK) return rc;
    hipLaunchKernelGGL(decode_kernel, dim3(a.total_tiles), dim3(kThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? ZC_OK : ZC_ERR_HIP;
}

extern "C" zc_status zc_decompress(const void *d_in, uint64_t in_bytes, uint64_t n, void *d_out, int32_t *d_status,
                                   void *stream) {
    zc_dec_seg s;
    s.in = d_in;
    s.in_bytes = in_bytes;
    s.n = n;
    s.out = d_out;
    s.status = d_status;
    return zc_decompress_batch(&s, 1, stream);
}

static uint32_t rd32(const uint8_t *p) {
    uint32_t v;
    std::memcpy(&v, p, 4);
    return v;
}
static uint64_t rd64(const uint8_t *p) {
    uint64_t v;
    std::memcpy(&v, p, 8);
    return v;
}

extern "C" zc_status zc_read_header(const void *host_header, uint64_t len, zc_stream_info *out) {
    if (!host_header || !out) return ZC_ERR_INVALID_ARG;
    if (len < kHeaderBytes) return ZC_ERR_CORRUPT;
    const uint8_t *h = static_cast<const uint8_t *>(host_header);
    const uint64_t n = rd64(h + 8);
    if (rd32(h) != kMagic || rd32(h + 4) != ((uint32_t)kVersion | (kHeaderBytes << 16)) || n > kMaxElems ||
        rd32(h + 16) != kGroup)
        return ZC_ERR_CORRUPT;
    const Layout L = layout_for(n);
    zc_plan p;
    std::memcpy(p.exps, h + 24, 7);
    p.reserved = h[31];
    const uint64_t E = rd64(h + 32), total = rd64(h + 40);
    if (rd32(h + 20) != L.groups || !plan_ok(p) || E > n || total != L.off_zp + E) return ZC_ERR_CORRUPT;
    for (int i = 48; i < 128; ++i)
        if (h[i]) return ZC_ERR_CORRUPT;
    out->n = n;
    out->zero_points = E;
    out->total_bytes = total;
    out->groups = (uint32_t)L.groups;
    out->plan = p;
    return ZC_OK;
}

extern "C" const char *zc_status_string(zc_status s) {
    switch (s) {
        case ZC_OK: return "ok";
        case ZC_ERR_INVALID_ARG: return "invalid argument";
        case ZC_ERR_CAPACITY: return "output capacity below zc_max_compressed_bytes(n)";
        case ZC_ERR_MISALIGNED: return "misaligned buffer";
        case ZC_ERR_CORRUPT: return "corrupt stream";
        case ZC_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}
