// Practical bandwidth ceilings for the codec's access shapes on MI355X
// (gfx950), for the benchmark only: the codec library never calls these.
//
// Each kernel moves the bytes of one codec direction with the codec's own
// access geometry and none of its arithmetic, so the time it takes is what
// the memory system allows for that shape:
//   * copy: 16 KiB per 256-thread block, four 128-bit non-temporal loads in
//     flight per lane, then the four stores (the raw-stream copy);
//   * encode shape: per 8192-value tile (256 threads, 4 steps of 8 values per
//     lane) 16 KiB read with 128-bit non-temporal loads, 8 KiB written with
//     8-byte stores (the sign+mantissa section) and 3 KiB with one dword per
//     thread in each of three regions (the code planes): 2 B read and
//     1.375 B written per value;
//   * decode shape: the mirror image, 8-byte and dword loads, 128-bit
//     non-temporal stores: 1.375 B read and 2 B written per value.
// The written words are cheap functions of every loaded word, so no load is
// dead.  n must be a multiple of 8192 (the benchmark sizes are).
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace zcb {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr uint32_t kTile = 8192;

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4 *in, u32x4 *out, uint64_t units) {
    const uint64_t base = (uint64_t)blockIdx.x * 4 * kThreads + threadIdx.x;
    u32x4 v[4];
#pragma unroll
    for (uint32_t u = 0; u < 4; ++u)
        if (base + u * kThreads < units) v[u] = __builtin_nontemporal_load(in + base + u * kThreads);
#pragma unroll
    for (uint32_t u = 0; u < 4; ++u)
        if (base + u * kThreads < units) __builtin_nontemporal_store(v[u], out + base + u * kThreads);
}

// One block per tile, like the encoder.
__global__ __launch_bounds__(kThreads) void encode_shape_kernel(const uint16_t *in, uint8_t *sm, uint8_t *planes,
                                                                uint64_t n) {
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const uint64_t tile0 = (uint64_t)blockIdx.x * kTile;
    u32x4 v[4];
#pragma unroll
    for (uint32_t u = 0; u < 4; ++u)
        v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(in + tile0 + 512u * (wave * 4 + u) + 8u * lane));
    uint32_t acc = 0;
#pragma unroll
    for (uint32_t u = 0; u < 4; ++u) {
        const u32x2 w = {v[u].x ^ v[u].y, v[u].z ^ v[u].w};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2 *>(sm + tile0 + 512u * (wave * 4 + u) + 8u * lane));
        acc ^= v[u].x + v[u].w;
    }
    const uint64_t pl = tile0 / 8 + 4u * tid;  // one dword per thread in each plane region
    const uint64_t region = n / 8;
#pragma unroll
    for (uint32_t p = 0; p < 3; ++p)
        __builtin_nontemporal_store(acc + p, reinterpret_cast<uint32_t *>(planes + p * region + pl));
}

__global__ __launch_bounds__(kThreads) void decode_shape_kernel(const uint8_t *sm, const uint8_t *planes,
                                                                uint16_t *out, uint64_t n) {
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const uint64_t tile0 = (uint64_t)blockIdx.x * kTile;
    const uint64_t region = n / 8;
    const uint64_t pl = tile0 / 8 + 4u * tid;
    uint32_t p[3];
#pragma unroll
    for (uint32_t q = 0; q < 3; ++q)
        p[q] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(planes + q * region + pl));
    u32x2 s[4];
#pragma unroll
    for (uint32_t u = 0; u < 4; ++u)
        s[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(sm + tile0 + 512u * (wave * 4 + u) + 8u * lane));
    const uint32_t k = p[0] ^ p[1] ^ p[2];
#pragma unroll
    for (uint32_t u = 0; u < 4; ++u) {
        const u32x4 w = {s[u].x ^ k, s[u].y, s[u].x + k, s[u].y ^ k};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(out + tile0 + 512u * (wave * 4 + u) + 8u * lane));
    }
}

}  // namespace zcb

using namespace zcb;

static int launched() { return hipGetLastError() == hipSuccess ? 0 : 1; }

// bytes: a multiple of 16; pointers 16-byte aligned.
extern "C" int zcb_copy(const void *in, void *out, uint64_t bytes, void *stream) {
    (void)hipGetLastError();
    const uint64_t units = bytes / 16;
    const uint64_t blocks = (units + 4 * kThreads - 1) / (4 * kThreads);
    if (blocks == 0 || blocks > 0xFFFFFFFFull) return 1;
    hipLaunchKernelGGL(copy_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(in), static_cast<u32x4 *>(out), units);
    return launched();
}

// in: n values; sm: n bytes; planes: 3n/8 bytes.
extern "C" int zcb_encode_shape(const void *in, uint64_t n, void *sm, void *planes, void *stream) {
    if (n % kTile) return 1;
    (void)hipGetLastError();
    hipLaunchKernelGGL(encode_shape_kernel, dim3((uint32_t)(n / kTile)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint16_t *>(in),
                       static_cast<uint8_t *>(sm), static_cast<uint8_t *>(planes), n);
    return launched();
}

// sm: n bytes; planes: 3n/8 bytes; out: n values.
extern "C" int zcb_decode_shape(const void *sm, const void *planes, uint64_t n, void *out, void *stream) {
    if (n % kTile) return 1;
    (void)hipGetLastError();
    hipLaunchKernelGGL(decode_shape_kernel, dim3((uint32_t)(n / kTile)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint8_t *>(sm),
                       static_cast<const uint8_t *>(planes), static_cast<uint16_t *>(out), n);
    return launched();
}
