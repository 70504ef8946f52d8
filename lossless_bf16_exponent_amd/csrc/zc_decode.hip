// Decompress kernels and their C ABI (BF16 exponent-coding codec, MI355X /
// gfx950): the inverse of section 2.B of the ZipCCL explainer pages.  The
// decoder needs no scan across tiles: the table of zero-point counts per
// 4096-element group gives every block its slice of the zero-point array,
// which is staged in LDS and gathered by rank; codes become exponents through
// a byte shuffle with the stream's table.  A raw stream (the fallback form) is
// checked and copied.
#include <hip/hip_runtime.h>

#include <cstring>

#include "zc.h"
#include "zc_device.h"
#include "zc_format.h"
#include "zc_lane.h"

namespace zc {

struct DecSeg {
    const uint8_t *in;
    uint16_t *out;
    int32_t *status;
    uint64_t in_bytes;
    uint32_t n;
    uint32_t tile_begin;  // first flat block of this segment
};
static_assert(sizeof(DecSeg) == 40, "compact kernel arguments");

struct DecArgs {
    uint32_t k;
    uint32_t total_tiles;
    DecSeg seg[ZC_MAX_BATCH];
    uint32_t tile_begin[ZC_MAX_BATCH];  // seg[i].tile_begin, contiguous for the block -> segment lookup
};
static_assert(sizeof(DecArgs) + 256 <= 4096, "decompress arguments fit the kernarg segment");

// The decode segment holding grid block `flat`.
__device__ __forceinline__ uint32_t find_segment_dec(const DecArgs &a, uint32_t flat) {
    return count_at_or_below<ZC_MAX_BATCH>(a.tile_begin, a.k, flat);
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
// decoder
// ---------------------------------------------------------------------------


// Header of a stream of n values, coded or raw: all 32 words load at once
// (uniform, scalar loads) and every field is tested without short-circuiting,
// so that no test waits for the one before it (a reduce block checks k headers
// up front).  On success `raw` tells the mode; for a coded stream tbl_lo/tbl_hi
// hold the code -> exponent table for v_perm (byte 0, code 000, is a
// placeholder) and E the zero-point count.  A raw stream (the fallback) is the
// header and the n values unchanged: total_bytes = 128 + 2n; its exps and E
// describe the coded form that was not kept.

__device__ __forceinline__ bool header_ok(const uint8_t *in, uint64_t in_bytes, uint64_t n, const Layout &L,
                                          uint32_t &tbl_lo, uint32_t &tbl_hi, uint64_t &E, bool &raw) {
    // constant address space: scalar loads, which never wait behind the
    // vector loads in flight
    const_u32 *h = (const_u32 *)in;
    uint32_t w[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i] = h[i];
    uint32_t pad = 0;
#pragma unroll
    for (int i = 12; i < 32; ++i) pad |= w[i];
    E = w[8] | ((uint64_t)w[9] << 32);
    const uint64_t total = w[10] | ((uint64_t)w[11] << 32);
    const uint32_t h6 = w[6], h7 = w[7];
    const uint32_t e[7] = {h6 & 0xFFu, (h6 >> 8) & 0xFFu, (h6 >> 16) & 0xFFu, h6 >> 24,
                           h7 & 0xFFu, (h7 >> 8) & 0xFFu, (h7 >> 16) & 0xFFu};
    const uint32_t mode = h7 >> 24;
    raw = mode == kModeRaw;
    const bool sized = ((mode == kModeCoded) & (total == L.off_zp + E)) | (raw & (total == kHeaderBytes + 2 * n));
    bool ok = (w[0] == kMagic) & (w[1] == ((uint32_t)kVersion | (kHeaderBytes << 16))) & (w[2] == (uint32_t)n) &
              (w[3] == (uint32_t)(n >> 32)) & (w[4] == kGroup) & (w[5] == (uint32_t)L.groups) & sized &
              (E <= n) & (total <= in_bytes) & (pad == 0u);
#pragma unroll
    for (int k = 1; k < 7; ++k) ok = ok & (e[k] > e[k - 1]);
    tbl_lo = h6 << 8;
    tbl_hi = (h6 >> 24) | (h7 << 8);
    return ok;
}

__device__ __forceinline__ bool raw_header_ok(const uint8_t *in, uint64_t in_bytes, uint64_t n, const Layout &L) {
    uint32_t lo, hi;
    uint64_t E;
    bool raw;
    return header_ok(in, in_bytes, n, L, lo, hi, E, raw) & raw;
}

// Values [v0, v1) of a raw stream to out (v0 a multiple of 8; the whole block).
__device__ __forceinline__ void copy_raw(const uint8_t *in, uint16_t *out, uint64_t v0, uint64_t v1) {
    const uint16_t *src = reinterpret_cast<const uint16_t *>(in + kHeaderBytes);
    const uint64_t full = v0 + ((v1 - v0) & ~uint64_t(7));
    for (uint64_t v = v0 + 8u * threadIdx.x; v < full; v += 8u * kThreads) {
        const uint4 q = load_stream16(src + v);
        store_stream16(out + v, q.x, q.y, q.z, q.w);
    }
    for (uint64_t v = full + threadIdx.x; v < v1; v += kThreads) out[v] = src[v];
}

// A block decodes kSub consecutive tiles (its span).  Every plane and
// sign+mantissa load of the span, and the span's zero-point table entries,
// are issued before the header is checked (all of them lie inside the n-value
// layout, which the host has checked against in_bytes); the zero-point slice
// is then staged in LDS with dword loads and gathered by rank.  The one-tile
// form asks for eight waves per SIMD: it then keeps to 77 SGPRs (82 without
// the budget, which leaves room for seven blocks per CU, not eight).
template <int kSub>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kSub == 1 ? 8 : 1, 8))) void decode_kernel(
    DecArgs args) {
    constexpr uint32_t kSpan = kTile * kSub;
    constexpr int kSpanGroups = (int)(kSpan / kGroup);
    __shared__ uint32_t s_planes[kTile / 8];
    __shared__ uint32_t s_zp32[kSpan / 4 + 3];  // the span's zero-point bytes from a dword-aligned start
    __shared__ uint32_t s_wave_total[2][kWaves];    // (+ slack for the 3-dword reads of the gather)
    __shared__ uint2 s_sel[256];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const uint32_t flat = blockIdx.x;
    const uint32_t s = find_segment_dec(args, flat);
    const DecSeg &sg = args.seg[s];
    const uint32_t b = flat - sg.tile_begin;
    const uint64_t n = sg.n;
    const Layout L = layout_for(n);
    const uint8_t *const in = sg.in;
    const uint64_t span0 = (uint64_t)b * kSpan;

    // ---- data loads of the whole span
    uint32_t pw[kSub][3];
    uint32_t sm[kSub][kSteps][2], vmask[kSub][kSteps];
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) {
        const uint64_t tile0 = span0 + (uint64_t)sub * kTile;
        pw[sub][0] = pw[sub][1] = pw[sub][2] = 0;
        if (tile0 + 32u * (uint32_t)tid < n) {
            const uint64_t off = tile0 / 8 + 4u * (uint32_t)tid;
            pw[sub][0] = load_stream4(in + L.off_p0 + off);
            pw[sub][1] = load_stream4(in + L.off_p1 + off);
            pw[sub][2] = load_stream4(in + L.off_p2 + off);
        }
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            const uint64_t base = tile0 + 512u * (uint32_t)(wave * kSteps + u) + 8u * (uint32_t)lane;
            sm[sub][u][0] = sm[sub][u][1] = 0;
            vmask[sub][u] = 0;
            if (base < n) {
                const uint2 v = load_stream8(in + kHeaderBytes + base);
                sm[sub][u][0] = v.x;
                sm[sub][u][1] = v.y;
                vmask[sub][u] = base + 8 <= n ? 0xFFu : (1u << (uint32_t)(n - base)) - 1u;
            }
        }
    }

    // ---- the span's zero-point table entries
    const uint32_t *tab = reinterpret_cast<const uint32_t *>(in + L.off_tab);
    uint32_t z[kSpanGroups + 1];
#pragma unroll
    for (int j = 0; j <= kSpanGroups; ++j) {
        const uint64_t g = (uint64_t)b * kSpanGroups + j;
        z[j] = tab[g <= L.groups ? g : L.groups];
    }

    // ---- header: every block checks it, so a bad header stops all of them.
    // (Tested field by field: this keeps the table entries above on scalar
    // loads issued with the data loads; the checks overlap those loads.)
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
        // not a coded stream: the raw fallback form, or corrupt
        if (raw_header_ok(in, sg.in_bytes, n, L)) {
            copy_raw(in, sg.out, span0, min(span0 + kSpan, n));
            return;
        }
        if (tid == 0 && sg.status) *sg.status = ZC_ERR_CORRUPT;
        return;
    }
    // code -> exponent table for v_perm: byte 0 (code 000) is a placeholder
    const uint32_t tbl_lo = h6 << 8, tbl_hi = (h6 >> 24) | (h7 << 8);

    // ---- table consistency; clamp so that every read stays inside the stream
    const bool last = (b == dec_blocks(n, kSpan) - 1);
    bool bad = (b == 0 && z[0] != 0) || (last && z[kSpanGroups] != E);
#pragma unroll
    for (int j = 0; j <= kSpanGroups; ++j) {
        const uint32_t lo = j ? z[j - 1] : 0u;
        if (z[j] < lo || z[j] > E) bad = true;
        z[j] = z[j] < lo ? lo : (z[j] > E ? (uint32_t)E : z[j]);
    }
    if (z[kSpanGroups] - z[0] > kSpan) {
        bad = true;
#pragma unroll
        for (int j = 0; j <= kSpanGroups; ++j) z[j] = z[j] - z[0] > kSpan ? z[0] + kSpan : z[j];
    }

    // ---- stage the span's zero-point bytes: stream bytes [A0, A1)
    const uint64_t A0 = L.off_zp + z[0], A1 = L.off_zp + z[kSpanGroups];
    const uint64_t a0 = A0 & ~uint64_t(3), a1 = A1 & ~uint64_t(3);
    const uint32_t shift = (uint32_t)(A0 & 3u);
    const uint32_t ndw = (uint32_t)((a1 - a0) / 4);
    for (uint32_t i = tid; i < ndw; i += kThreads) s_zp32[i] = ld_u32(in + a0 + 4u * i);
    if (tid == 0 && A1 > a1) {
        uint32_t w = 0;
        for (uint32_t i = 0; i < (uint32_t)(A1 - a1); ++i) w |= (uint32_t)in[a1 + i] << (8 * i);
        s_zp32[ndw] = w;
    }
    const uint32_t zspan = z[kSpanGroups] - z[0];
    zp_selectors(s_sel);  // visible after the first sub-tile's barrier

#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) {
        const uint64_t tile0 = span0 + (uint64_t)sub * kTile;
        {
            const uint32_t p0 = pw[sub][0], p1 = pw[sub][1], p2 = pw[sub][2];
            const uint32_t lo = perm(p1, p0, 0x05010400u), hi = perm(p1, p0, 0x07030602u);
            uint4 q;
            q.x = perm(p2, lo, 0x0C040100u);
            q.y = perm(p2, lo, 0x0C050302u);
            q.z = perm(p2, hi, 0x0C060100u);
            q.w = perm(p2, hi, 0x0C070302u);
            reinterpret_cast<uint4 *>(s_planes)[tid] = q;
        }
        __syncthreads();  // s_planes (and, for the first sub-tile, s_zp32)

        uint32_t e[kSteps][2], zmask[kSteps];
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            const uint32_t planes = s_planes[(wave * kSteps + u) * kWave + lane] & 0x00FFFFFFu;
            uint32_t c_lo, c_hi;
            planes_to_codes(planes, c_lo, c_hi);
            e[u][0] = perm(tbl_hi, tbl_lo, c_lo);
            e[u][1] = perm(tbl_hi, tbl_lo, c_hi);
            zmask[u] = zero_point_mask(planes) & vmask[sub][u];
        }
        const TileCounts tc = count_tile(zmask, lane, wave, s_wave_total[sub & 1]);
        const uint32_t zb = z[2 * sub], zm = z[2 * sub + 1], ze = z[2 * sub + 2];
        if (tc.tile_total != ze - zb || tc.first_group != zm - zb) bad = true;

        const uint32_t rank0 = zb - z[0];
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            // slice byte j sits at byte shift + j of s_zp32; a rank past the
            // slice (a corrupt table, already flagged) reads the slack instead
            const uint32_t rk = rank0 + tc.rank[u];
            put_zero_points(e[u][0], e[u][1], zmask[u], shift + (rk <= zspan ? rk : zspan), s_zp32, s_sel);
            const uint64_t base = tile0 + 512u * (uint32_t)(wave * kSteps + u) + 8u * (uint32_t)lane;
            uint32_t o0, o1, o2, o3;
            rebuild4(sm[sub][u][0], e[u][0], o0, o1);
            rebuild4(sm[sub][u][1], e[u][1], o2, o3);
            if (vmask[sub][u] == 0xFFu) {
                store_stream16(sg.out + base, o0, o1, o2, o3);
            } else if (vmask[sub][u]) {
                const uint32_t w4[4] = {o0, o1, o2, o3};
                for (uint32_t i = 0; base + i < n; ++i) sg.out[base + i] = (uint16_t)(w4[i / 2] >> (16 * (i % 2)));
            }
        }
        if (sub + 1 < kSub) __syncthreads();  // s_planes is rewritten by the next sub-tile
    }
    if (bad && tid == 0 && sg.status) atomicMax(sg.status, (int32_t)ZC_ERR_CORRUPT);
}

// Segments whose buffer is shorter than the coded layout of n values can only
// hold a raw stream: checked and copied without any read at a coded offset.
__global__ __launch_bounds__(kThreads) void decode_raw_kernel(DecArgs args) {
    const uint32_t flat = blockIdx.x;
    const uint32_t s = find_segment_dec(args, flat);
    const DecSeg &sg = args.seg[s];
    const uint64_t n = sg.n;
    const Layout L = layout_for(n);
    const uint64_t span0 = (uint64_t)(flat - sg.tile_begin) * kDecRawSpan;
    if (!raw_header_ok(sg.in, sg.in_bytes, n, L)) {
        if (threadIdx.x == 0 && sg.status) *sg.status = ZC_ERR_CORRUPT;
        return;
    }
    copy_raw(sg.in, sg.out, span0, min(span0 + kDecRawSpan, n));
}

}  // namespace zc

// ===========================================================================
// C ABI
// ===========================================================================

using namespace zc;

zc_status zc::launch_zero(ZeroArgs &z, hipStream_t st) {
    uint64_t words = 0;
    for (uint32_t i = 0; i < z.count; ++i) words += z.r[i].words;
    if (!words) return ZC_OK;
    uint64_t blocks = (words + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(zero_kernel, dim3((uint32_t)blocks), dim3(256), 0, st, z);
    return hipGetLastError() == hipSuccess ? ZC_OK : ZC_ERR_HIP;
}

extern "C" zc_status zc_decompress_batch(const zc_dec_seg *segs, uint32_t k, void *stream) {
    if (!segs || k == 0 || k > ZC_MAX_BATCH) return ZC_ERR_INVALID_ARG;
    // a[0]: decode_kernel; a[1]: decode_raw_kernel, for buffers shorter than
    // the coded layout (only a raw stream fits there)
    DecArgs a[2];
    std::memset(a, 0, sizeof(a));
    ZeroArgs z;
    std::memset(&z, 0, sizeof(z));
    uint64_t tiles[2] = {0, 0};
    // the decode_kernel launch's span: one tile for a launch of at least
    // kDecNarrowMin values or at most kDecNarrowMax, else two
    // (decode_raw_kernel keeps two)
    uint64_t coded_values = 0;
    for (uint32_t i = 0; i < k; ++i) {
        const zc_dec_seg &g = segs[i];
        if (!g.in || g.n > kMaxElems || (g.n && !g.out)) return ZC_ERR_INVALID_ARG;
        if (((uintptr_t)g.in & 127u) || ((uintptr_t)g.out & 15u) || ((uintptr_t)g.status & 3u))
            return ZC_ERR_MISALIGNED;
        const Layout L = layout_for(g.n);
        // no stream of n values is shorter than both forms
        if (g.in_bytes < L.off_zp && g.in_bytes < kHeaderBytes + 2 * g.n) return ZC_ERR_CORRUPT;
        if (g.in_bytes >= L.off_zp) coded_values += g.n;
    }
    const bool narrow = coded_values >= kDecNarrowMin || coded_values <= kDecNarrowMax;
    const uint32_t span[2] = {narrow ? kTile : kTile * kDecWideTiles, kDecRawSpan};
    for (uint32_t i = 0; i < k; ++i) {
        const zc_dec_seg &g = segs[i];
        const Layout L = layout_for(g.n);
        const int which = g.in_bytes < L.off_zp ? 1 : 0;
        DecSeg &d = a[which].seg[a[which].k++];
        d.in = static_cast<const uint8_t *>(g.in);
        d.out = static_cast<uint16_t *>(g.out);
        d.status = g.status;
        d.in_bytes = g.in_bytes;
        d.n = (uint32_t)g.n;
        d.tile_begin = (uint32_t)tiles[which];
        a[which].tile_begin[a[which].k - 1] = d.tile_begin;
        tiles[which] += dec_blocks(g.n, span[which]);
        if (tiles[which] > 0xFFFFFFFFull) return ZC_ERR_INVALID_ARG;
        if (g.status) {
            z.r[z.count].ptr = reinterpret_cast<uint32_t *>(g.status);
            z.r[z.count].words = 1;
            ++z.count;
        }
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    zc_status rc = launch_zero(z, st);
    if (rc != ZC_OK) return rc;
    for (int which = 0; which < 2; ++which) {
        if (!a[which].k) continue;
        a[which].total_tiles = (uint32_t)tiles[which];
        if (which == 0 && narrow)
            hipLaunchKernelGGL(decode_kernel<1>, dim3(a[0].total_tiles), dim3(kThreads), 0, st, a[0]);
        else if (which == 0)
            hipLaunchKernelGGL(decode_kernel<kDecWideTiles>, dim3(a[0].total_tiles), dim3(kThreads), 0, st, a[0]);
        else
            hipLaunchKernelGGL(decode_raw_kernel, dim3(a[1].total_tiles), dim3(kThreads), 0, st, a[1]);
        if (hipGetLastError() != hipSuccess) return ZC_ERR_HIP;
    }
    return ZC_OK;
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
