// Online statistics of a BF16 tensor on MI355X (gfx950): the exponent
// histogram with its top-7 table, and a sigma estimate for the closed-form
// table.
//
// The ZipCCL explainer pages ("ZipCCL: Efficient Lossless Data Compression of
// Communication Collectives for Accelerating LLM Training", section 2.A)
// derive the table of the seven frequent exponents from the standard
// deviation of the tensor instead of building a histogram or sorting online.
// These calls are that online path, so that the two can be compared and so
// that a caller without a trusted sigma can still get a table:
//   * zc_exponent_histogram counts every exponent field (bits 14..7);
//     zc_plan_from_histogram (host) takes its seven largest counts;
//   * zc_estimate_sigma returns the root mean square of the finite values (the
//     maximum-likelihood sigma of the zero-mean Gaussian the pages assume),
//     which zc_plan_from_sigma turns into the closed-form table.
//
// Design on gfx950 (both passes are HBM-bound streaming reads, no MFMA):
//   * Histogram: a 512-thread block keeps 64 lane-private columns of the 256
//     bins in LDS (64 KiB, bin-major, lane-minor), so the LDS add of lane l
//     always hits bank l whatever the data: the heavy concentration of the
//     exponents (a few fields hold most values) costs no bank conflicts and no
//     same-address serialization.  The 8 waves of a block share the columns
//     through LDS atomics without return.  Two blocks fill a CU.  Each block
//     writes its 256 counts to a row of the workspace; a second small kernel
//     (one block per bin) sums the columns.  No global atomics (same-address device atomics
//     serialize behind a round trip each).
//   * Sigma: float64 sums of exact squares (a BF16 square has 16 significant
//     bits and stays inside the double range), per thread in element order,
//     then fixed-order trees in the block and in a one-block final kernel.
//     The grid size is fixed, so the result depends only on the input.
//   * Both read 128-bit nontemporal loads, two tiles in flight per thread
//     (two register sets in turn).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "zc.h"

namespace zcs {

constexpr uint64_t kMaxElems = 0xFFFFFFFFull;

// Histogram pass geometry.
constexpr int kHistThreads = 512;
constexpr int kHistChunks = 4;  // 16-byte loads per thread per tile
constexpr uint64_t kHistTileChunks = (uint64_t)kHistThreads * kHistChunks;  // 2048 chunks = 16384 values
constexpr uint32_t kHistBlocks = 512;                                       // two per CU on 256 CUs
constexpr int kBins = 256;
constexpr int kCols = 64;  // one LDS column per lane

// Sigma pass geometry.
constexpr int kSigThreads = 256;
constexpr int kSigChunks = 4;
constexpr uint64_t kSigTileChunks = (uint64_t)kSigThreads * kSigChunks;  // 1024 chunks = 8192 values
constexpr uint32_t kSigBlocks = 2048;

// Workspace: the histogram rows (u32 [kHistBlocks][256]) or the sigma
// partials ({double, u64} [kSigBlocks]); one call uses one of the two.
constexpr uint64_t kHistRowsBytes = (uint64_t)kHistBlocks * kBins * 4;
constexpr uint64_t kSigPartBytes = (uint64_t)kSigBlocks * 16;
constexpr uint64_t kWorkspaceBytes = kHistRowsBytes > kSigPartBytes ? kHistRowsBytes : kSigPartBytes;

__device__ __forceinline__ uint4 load_nt(const uint4 *p) {
    uint4 v;
    v.x = __builtin_nontemporal_load(&p->x);
    v.y = __builtin_nontemporal_load(&p->y);
    v.z = __builtin_nontemporal_load(&p->z);
    v.w = __builtin_nontemporal_load(&p->w);
    return v;
}

// ---------------------------------------------------------------------------
// exponent histogram
// ---------------------------------------------------------------------------

struct HistArgs {
    const uint16_t *in;
    uint64_t n;
    uint32_t *rows;  // [kHistBlocks][256]
};

__device__ __forceinline__ void lds_count(uint32_t *cols, uint32_t field, uint32_t lane) {
    __hip_atomic_fetch_add(cols + field * kCols + lane, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void count_word(uint32_t *cols, uint32_t w, uint32_t lane) {
    lds_count(cols, (w >> 7) & 0xFFu, lane);
    lds_count(cols, (w >> 23) & 0xFFu, lane);
}

__device__ __forceinline__ void count_chunk(uint32_t *cols, const uint4 &v, uint32_t lane) {
    count_word(cols, v.x, lane);
    count_word(cols, v.y, lane);
    count_word(cols, v.z, lane);
    count_word(cols, v.w, lane);
}

// A chunk past the end goes to the spare bin kBins, so that every loaded value
// is consumed on every path (a skipped load would still be pending at the
// top of the loop, where its registers are reused, and force a full wait).
__device__ __forceinline__ void count_chunk_masked(uint32_t *cols, const uint4 &v, uint32_t lane, bool valid) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lds_count(cols, valid ? (w[i] >> 7) & 0xFFu : (uint32_t)kBins, lane);
        lds_count(cols, valid ? (w[i] >> 23) & 0xFFu : (uint32_t)kBins, lane);
    }
}

__global__ __launch_bounds__(kHistThreads) void hist_kernel(HistArgs a) {
    __shared__ uint32_t cols[(kBins + 1) * kCols];  // 64 KiB and a spare bin
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kCols - 1);
    {
        uint4 *c4 = reinterpret_cast<uint4 *>(cols);
        for (uint32_t i = tid; i < kBins * kCols / 4; i += kHistThreads) c4[i] = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();

    const uint4 *in4 = reinterpret_cast<const uint4 *>(a.in);
    const uint64_t chunks = a.n / 8;  // whole 16-byte chunks
    const uint64_t tiles = (chunks + kHistTileChunks - 1) / kHistTileChunks;
    // Two register sets in turn, so the loads of the next tile are in flight
    // while this one is counted.  Loads are unconditional (a chunk index past
    // the end is clamped to the last chunk, whose value is then not counted),
    // which keeps the issue free of branches.
    auto fetch = [&](uint64_t t, uint4 *dst) {
#pragma unroll
        for (int q = 0; q < kHistChunks; ++q) {
            uint64_t c = t * kHistTileChunks + (uint64_t)q * kHistThreads + tid;
            c = c < chunks ? c : chunks - 1;
            dst[q] = load_nt(in4 + c);
        }
        __builtin_amdgcn_sched_barrier(0);  // issue these loads before counting the previous tile
    };
    auto count = [&](uint64_t t, const uint4 *v) {
        if ((t + 1) * kHistTileChunks <= chunks) {
#pragma unroll
            for (int q = 0; q < kHistChunks; ++q) count_chunk(cols, v[q], lane);
        } else {
#pragma unroll
            for (int q = 0; q < kHistChunks; ++q)
                count_chunk_masked(cols, v[q], lane, t * kHistTileChunks + (uint64_t)q * kHistThreads + tid < chunks);
        }
    };
    // tiles blockIdx.x + i * kHistBlocks, i = 0 .. iters-1, two per round
    const uint64_t first = blockIdx.x;
    const uint64_t iters = first < tiles ? (tiles - first + kHistBlocks - 1) / kHistBlocks : 0;
    if (iters) {
        uint4 va[kHistChunks], vb[kHistChunks];
        fetch(first, va);
        uint64_t i = 0;
        for (; i + 2 <= iters; i += 2) {
            const uint64_t t = first + i * kHistBlocks;
            fetch(t + kHistBlocks, vb);
            count(t, va);
            fetch(t + 2 * kHistBlocks, va);  // past the last tile: every lane reads the last chunk
            count(t + kHistBlocks, vb);
        }
        if (i < iters) count(first + i * kHistBlocks, va);
    }
    // the last n mod 8 values (fewer than one chunk), counted by block 0
    if (blockIdx.x == 0 && tid < (a.n & 7u)) lds_count(cols, ((uint32_t)a.in[chunks * 8 + tid] >> 7) & 0xFFu, lane);
    __syncthreads();

    // bin b = tid / 2 sums 32 of its 64 columns (half tid & 1); the start is
    // rotated by the bin so that the 32 bins of a wave read 32 distinct banks
    const uint32_t bin = tid >> 1, half = tid & 1u;
    uint32_t s = 0;
#pragma unroll 8
    for (uint32_t j = 0; j < 32; ++j) s += cols[bin * kCols + ((half * 32 + j + bin) & (kCols - 1))];
    s += __shfl_xor(s, 1);
    if (!half) a.rows[(uint64_t)blockIdx.x * kBins + bin] = s;
}

// hist[b] = sum over the rows of column b: one block per bin, every thread
// adds kHistBlocks / 256 rows with all of its loads in flight at once (the
// pass is a single round trip; the rows' cache lines are shared by the
// blocks of 16 neighbouring bins).
struct HistSumArgs {
    const uint32_t *rows;
    unsigned long long *hist;
};

constexpr int kSumThreads = 256;
static_assert(kHistBlocks % kSumThreads == 0, "whole rows per thread");

__global__ __launch_bounds__(kSumThreads) void hist_sum_kernel(HistSumArgs a) {
    __shared__ unsigned long long part[kSumThreads / 64];
    const uint32_t tid = threadIdx.x, bin = blockIdx.x;
    uint32_t v[kHistBlocks / kSumThreads];
#pragma unroll
    for (uint32_t i = 0; i < kHistBlocks / kSumThreads; ++i) v[i] = a.rows[(uint64_t)(tid + i * kSumThreads) * kBins + bin];
    unsigned long long s = 0;
#pragma unroll
    for (uint32_t i = 0; i < kHistBlocks / kSumThreads; ++i) s += v[i];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    if ((tid & 63u) == 0) part[tid >> 6] = s;
    __syncthreads();
    if (tid == 0) a.hist[bin] = part[0] + part[1] + part[2] + part[3];
}

// ---------------------------------------------------------------------------
// sigma estimate
// ---------------------------------------------------------------------------

struct SigArgs {
    const uint16_t *in;
    uint64_t n;
    double *part_sum;                 // [kSigBlocks]
    unsigned long long *part_count;   // [kSigBlocks]
};

// x^2 of both BF16 halves of a word, NaN and Inf (field 255) excluded.
__device__ __forceinline__ void square_word(uint32_t w, double &acc, uint32_t &cnt) {
    const uint32_t lo = w << 16, hi = w & 0xFFFF0000u;
    const bool flo = ((lo >> 23) & 0xFFu) != 0xFFu, fhi = ((hi >> 23) & 0xFFu) != 0xFFu;
    const double xlo = flo ? (double)__uint_as_float(lo) : 0.0;
    const double xhi = fhi ? (double)__uint_as_float(hi) : 0.0;
    acc = fma(xlo, xlo, acc);
    acc = fma(xhi, xhi, acc);
    cnt += (uint32_t)flo + (uint32_t)fhi;
}

// Fast path for a chunk whose 8 values are all finite (the usual case).
__device__ __forceinline__ bool chunk_finite(const uint4 &v) {
    // a half is non-finite when its 8 exponent bits are all ones
    auto bad = [](uint32_t w) { return ((w & 0x7F80u) == 0x7F80u) | ((w & 0x7F800000u) == 0x7F800000u); };
    return !(bad(v.x) | bad(v.y) | bad(v.z) | bad(v.w));
}

__device__ __forceinline__ void square_chunk(const uint4 &v, double &acc, uint32_t &cnt) {
    if (chunk_finite(v)) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double xlo = (double)__uint_as_float(w[i] << 16);
            const double xhi = (double)__uint_as_float(w[i] & 0xFFFF0000u);
            acc = fma(xlo, xlo, acc);
            acc = fma(xhi, xhi, acc);
        }
        cnt += 8;
    } else {
        square_word(v.x, acc, cnt);
        square_word(v.y, acc, cnt);
        square_word(v.z, acc, cnt);
        square_word(v.w, acc, cnt);
    }
}

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ unsigned long long wave_sum(unsigned long long x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__global__ __launch_bounds__(kSigThreads) void sigma_kernel(SigArgs a) {
    __shared__ double ssum[kSigThreads / 64];
    __shared__ unsigned long long scnt[kSigThreads / 64];
    const uint32_t tid = threadIdx.x;
    const uint4 *in4 = reinterpret_cast<const uint4 *>(a.in);
    const uint64_t chunks = a.n / 8;
    const uint64_t tiles = (chunks + kSigTileChunks - 1) / kSigTileChunks;
    double acc = 0.0;
    uint32_t cnt = 0;
    auto fetch = [&](uint64_t t, uint4 *dst) {
#pragma unroll
        for (int q = 0; q < kSigChunks; ++q) {
            uint64_t c = t * kSigTileChunks + (uint64_t)q * kSigThreads + tid;
            c = c < chunks ? c : chunks - 1;
            dst[q] = load_nt(in4 + c);
        }
        __builtin_amdgcn_sched_barrier(0);  // issue these loads before adding the previous tile
    };
    // a chunk past the end is replaced by zeros (adding 0 to the sum exactly)
    // and taken back out of the count, so every loaded value is consumed on
    // every path and no load is left pending where its registers are reused
    auto add = [&](uint64_t t, const uint4 *v) {
#pragma unroll
        for (int q = 0; q < kSigChunks; ++q) {
            const bool valid = t * kSigTileChunks + (uint64_t)q * kSigThreads + tid < chunks;
            square_chunk(valid ? v[q] : make_uint4(0, 0, 0, 0), acc, cnt);
            cnt -= valid ? 0u : 8u;
        }
    };
    const uint64_t first = blockIdx.x;
    const uint64_t iters = first < tiles ? (tiles - first + kSigBlocks - 1) / kSigBlocks : 0;
    if (iters) {
        uint4 va[kSigChunks], vb[kSigChunks];
        fetch(first, va);
        uint64_t i = 0;
        for (; i + 2 <= iters; i += 2) {
            const uint64_t t = first + i * kSigBlocks;
            fetch(t + kSigBlocks, vb);
            add(t, va);
            fetch(t + 2 * kSigBlocks, va);  // past the last tile: every lane reads the last chunk
            add(t + kSigBlocks, vb);
        }
        if (i < iters) add(first + i * kSigBlocks, va);
    }
    // the last n mod 8 values, added by block 0
    if (blockIdx.x == 0 && tid < (a.n & 7u)) {
        const uint32_t w = (uint32_t)a.in[chunks * 8 + tid] << 16;
        if (((w >> 23) & 0xFFu) != 0xFFu) {
            const double x = (double)__uint_as_float(w);
            acc = fma(x, x, acc);
            cnt += 1;
        }
    }
    const double ws = wave_sum(acc);
    const unsigned long long wc = wave_sum((unsigned long long)cnt);
    if ((tid & 63u) == 0) {
        ssum[tid >> 6] = ws;
        scnt[tid >> 6] = wc;
    }
    __syncthreads();
    if (tid == 0) {
        a.part_sum[blockIdx.x] = (ssum[0] + ssum[1]) + (ssum[2] + ssum[3]);
        a.part_count[blockIdx.x] = scnt[0] + scnt[1] + scnt[2] + scnt[3];
    }
}

struct SigFinalArgs {
    const double *part_sum;
    const unsigned long long *part_count;
    double *sigma;
    unsigned long long *finite;  // nullable
};

__global__ __launch_bounds__(256) void sigma_final_kernel(SigFinalArgs a) {
    __shared__ double ssum[4];
    __shared__ unsigned long long scnt[4];
    const uint32_t tid = threadIdx.x;
    double ps[kSigBlocks / 256];
    unsigned long long pc[kSigBlocks / 256];
#pragma unroll
    for (uint32_t i = 0; i < kSigBlocks / 256; ++i) {  // every load in flight at once
        ps[i] = a.part_sum[tid + 256 * i];
        pc[i] = a.part_count[tid + 256 * i];
    }
    double s = 0.0;
    unsigned long long c = 0;
#pragma unroll
    for (uint32_t i = 0; i < kSigBlocks / 256; ++i) {
        s += ps[i];
        c += pc[i];
    }
    s = wave_sum(s);
    c = wave_sum(c);
    if ((tid & 63u) == 0) {
        ssum[tid >> 6] = s;
        scnt[tid >> 6] = c;
    }
    __syncthreads();
    if (tid == 0) {
        const double sum = (ssum[0] + ssum[1]) + (ssum[2] + ssum[3]);
        const unsigned long long count = scnt[0] + scnt[1] + scnt[2] + scnt[3];
        *a.sigma = count ? sqrt(sum / (double)count) : 0.0;
        if (a.finite) *a.finite = count;
    }
}

}  // namespace zcs

// ===========================================================================
// C ABI
// ===========================================================================

using namespace zcs;

extern "C" uint64_t zc_stats_workspace_bytes(uint64_t n) { return n > kMaxElems ? 0 : kWorkspaceBytes; }

static zc_status check_stats_args(const void *d_in, uint64_t n, const void *d_ws, uint64_t ws_bytes,
                                  const void *d_out) {
    if (n > kMaxElems || !d_out || !d_ws || (n && !d_in)) return ZC_ERR_INVALID_ARG;
    if (((uintptr_t)d_in & 15u) || ((uintptr_t)d_ws & 15u) || ((uintptr_t)d_out & 7u)) return ZC_ERR_MISALIGNED;
    if (ws_bytes < kWorkspaceBytes) return ZC_ERR_CAPACITY;
    return ZC_OK;
}

// The two histogram launches over a workspace of kWorkspaceBytes at `rows`.
// Every block of hist_kernel writes its whole row (also with no tile, n = 0
// included) and hist_sum_kernel reads only those rows, so the workspace never
// needs clearing.
static zc_status launch_histogram(const void *d_in, uint64_t n, uint32_t *rows, uint64_t *d_hist, hipStream_t st) {
    (void)hipGetLastError();
    HistArgs h;
    h.in = static_cast<const uint16_t *>(d_in);
    h.n = n;
    h.rows = rows;
    hipLaunchKernelGGL(hist_kernel, dim3(kHistBlocks), dim3(kHistThreads), 0, st, h);
    if (hipGetLastError() != hipSuccess) return ZC_ERR_HIP;
    HistSumArgs s;
    s.rows = rows;
    s.hist = reinterpret_cast<unsigned long long *>(d_hist);
    hipLaunchKernelGGL(hist_sum_kernel, dim3(kBins), dim3(kSumThreads), 0, st, s);
    return hipGetLastError() == hipSuccess ? ZC_OK : ZC_ERR_HIP;
}

extern "C" zc_status zc_exponent_histogram(const void *d_in, uint64_t n, void *d_workspace, uint64_t workspace_bytes,
                                           uint64_t *d_hist, void *stream) {
    const zc_status rc = check_stats_args(d_in, n, d_workspace, workspace_bytes, d_hist);
    if (rc != ZC_OK) return rc;
    return launch_histogram(d_in, n, static_cast<uint32_t *>(d_workspace), d_hist, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// The histogram without a caller workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops that forbid
// hipMalloc).  The workspace is this file-scope device array: every GPU that
// runs the call holds one copy of it until the process ends.  Host code never
// uses the array's name as an address (on the host it is only a stand-in for
// the symbol): the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current.
// ---------------------------------------------------------------------------

static __device__ __align__(256) uint8_t scratch[kWorkspaceBytes];

constexpr int kMaxDevices = 64;
static std::atomic<void *> g_scratch[kMaxDevices];
static std::mutex g_scratch_mutex;

// The current device's copy of `scratch`, looked up on the first call on that
// device; NULL when HIP cannot report it.
static void *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) {
            (void)hipGetLastError();
            return nullptr;
        }
        p = q;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

extern "C" zc_status zc_exponent_histogram_noalloc(const void *d_in, uint64_t n, uint64_t *d_hist, void *stream) {
    if (n > kMaxElems || !d_hist || (n && !d_in)) return ZC_ERR_INVALID_ARG;
    if (((uintptr_t)d_in & 15u) || ((uintptr_t)d_hist & 7u)) return ZC_ERR_MISALIGNED;
    void *ws = device_scratch();
    if (!ws) return ZC_ERR_HIP;
    return launch_histogram(d_in, n, static_cast<uint32_t *>(ws), d_hist, static_cast<hipStream_t>(stream));
}

extern "C" zc_status zc_estimate_sigma(const void *d_in, uint64_t n, void *d_workspace, uint64_t workspace_bytes,
                                       double *d_sigma, uint64_t *d_finite, void *stream) {
    zc_status rc = check_stats_args(d_in, n, d_workspace, workspace_bytes, d_sigma);
    if (rc != ZC_OK) return rc;
    if ((uintptr_t)d_finite & 7u) return ZC_ERR_MISALIGNED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    SigArgs a;
    a.in = static_cast<const uint16_t *>(d_in);
    a.n = n;
    a.part_sum = static_cast<double *>(d_workspace);
    a.part_count = reinterpret_cast<unsigned long long *>(static_cast<uint8_t *>(d_workspace) + kSigBlocks * 8);
    hipLaunchKernelGGL(sigma_kernel, dim3(kSigBlocks), dim3(kSigThreads), 0, st, a);
    if (hipGetLastError() != hipSuccess) return ZC_ERR_HIP;
    SigFinalArgs f;
    f.part_sum = a.part_sum;
    f.part_count = a.part_count;
    f.sigma = d_sigma;
    f.finite = reinterpret_cast<unsigned long long *>(d_finite);
    hipLaunchKernelGGL(sigma_final_kernel, dim3(1), dim3(256), 0, st, f);
    return hipGetLastError() == hipSuccess ? ZC_OK : ZC_ERR_HIP;
}
