// Device helpers shared by the codec's kernels on MI355X (gfx950): streaming
// loads and stores, wave-wide scans, the zero-point gather of the decoders,
// and the argument block of the small fill kernel.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "zc.h"
#include "zc_format.h"
#include "zc_lane.h"

namespace zc {

struct ZeroRegion {
    uint32_t *ptr;
    uint64_t words;
};

struct ZeroArgs {
    uint32_t count;
    ZeroRegion r[ZC_MAX_BATCH];
};

// Clears each region (the decoders' status words) in one small launch.
zc_status launch_zero(ZeroArgs &z, hipStream_t st);

// ---------------------------------------------------------------------------
// streaming memory access: every codec byte is read once and written once,
// so loads and stores carry the non-temporal hint (measured on MI355X: a
// 128-bit copy moves 13 % more bytes per second with it)
// ---------------------------------------------------------------------------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2a4 __attribute__((ext_vector_type(2), aligned(4)));  // 8 bytes, dword-aligned
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));  // 16 bytes, dword-aligned
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

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS):
// shifts of 1, 2, 4 and 8 lanes inside each 16-lane row, then the last lane
// of row 0 / row 2 is broadcast into rows 1 / 3 and lane 31 into rows 2 and 3.
// A lane whose source lies outside its row keeps the 0 passed as `old`.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return v;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan(v), kWave - 1);
}

// How many of v[1 .. count) are at or below flat, for non-decreasing v: the
// index of the last entry at or below it.  Lane i reads entries 1 + i,
// 65 + i, ... with one vector load per 64 entries and a ballot counts the
// hits, so the lookup costs one round trip whatever the count (a loop of
// dependent reads, one per entry or per halving, cost a decoder block 32 of
// them at its start, 7 % of the bucket's decompress time).  All lanes of the
// wave must be active.
template <uint32_t kEntries>
__device__ __forceinline__ uint32_t count_at_or_below(const uint32_t *v, uint32_t count, uint32_t flat,
                                                      uint32_t mask = ~0u) {
    const uint32_t lane = __lane_id();
    uint32_t total = 0;
#pragma unroll
    for (uint32_t c = 0; c < (kEntries - 1 + kWave - 1) / kWave; ++c) {
        const uint32_t i = 1u + (uint32_t)kWave * c + lane;
        const bool hit = i < count && (v[i] & mask) <= flat;  // (read only below count: inside the array)
        total += (uint32_t)__builtin_popcountll(__ballot(hit));
    }
    return total;
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
    const uint32_t ai = wave_inclusive_scan(a), bi = wave_inclusive_scan(b);
    const uint32_t at = (uint32_t)__builtin_amdgcn_readlane((int)ai, kWave - 1);
    const uint32_t bt = (uint32_t)__builtin_amdgcn_readlane((int)bi, kWave - 1);
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

typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;
// Constant address space: loads through it are scalar loads.
typedef __attribute__((address_space(4))) const uint32_t const_u32;

__device__ __forceinline__ uint32_t ld_u32(const uint8_t *p) { return *reinterpret_cast<const uint32_t *>(p); }

// Gather of the zero-point bytes of an 8-value step without a loop: the
// step's zero-points are the bytes [r, r + popcount(m)) of the slice, in
// order.  sel[m] holds, for each of the 8 positions, the index among the set
// bits of m (a v_perm selector into those bytes) or 0x0C (a zero byte) where
// the bit is clear; the same selector applied to all-ones bytes gives the
// byte mask of the positions to replace.
__device__ __forceinline__ void zp_selectors(uint2 *sel) {  // 256 entries, filled by the block
    for (uint32_t m = threadIdx.x; m < 256; m += kThreads) {
        uint32_t lo = 0, hi = 0, idx = 0;
        for (uint32_t p = 0; p < 8; ++p) {
            const uint32_t b = (m >> p) & 1u ? idx++ : 0x0Cu;
            if (p < 4)
                lo |= b << (8 * p);
            else
                hi |= b << (8 * (p - 4));
        }
        sel[m] = make_uint2(lo, hi);
    }
}

__device__ __forceinline__ void put_zero_points(uint32_t &e_lo, uint32_t &e_hi, uint32_t m, uint32_t r,
                                                const uint32_t *zw, const uint2 *sel) {
    const uint32_t d0 = zw[r / 4], d1 = zw[r / 4 + 1], d2 = zw[r / 4 + 2];
    const uint32_t sh = r & 3u;
    const uint32_t z_lo = __builtin_amdgcn_alignbyte(d1, d0, sh), z_hi = __builtin_amdgcn_alignbyte(d2, d1, sh);
    const uint2 s = sel[m];
    e_lo = bfi(perm(~0u, ~0u, s.x), perm(z_hi, z_lo, s.x), e_lo);
    e_hi = bfi(perm(~0u, ~0u, s.y), perm(z_hi, z_lo, s.y), e_hi);
}

}  // namespace zc
