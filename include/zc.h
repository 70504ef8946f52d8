/*
 * zc.h -- C ABI of the MI355X (gfx950) BF16 exponent-coding codec.
 *
 * The method is the exponent coding described on the explainer pages of
 *   "ZipCCL: Efficient Lossless Data Compression of Communication Collectives
 *    for Accelerating LLM Training" (gist.science; fr / ja / ko pages),
 * technical summary, section 2 ("Methodology"):
 *   2.A  near-Gaussian training tensors concentrate their BF16 exponents; the
 *        7 most frequent cover more than 97 % of the values, and the table of
 *        those 7 is derived from the standard deviation sigma instead of an
 *        online histogram or sort;
 *   2.B  each value is split into sign+mantissa bits and exponent bits; an
 *        exponent among the 7 becomes a 3-bit code 001..111, any other gets the
 *        "zero-point" code 000 and its full 8 bits go to a separate zero-point
 *        array; 16 bits become 11 when no value takes the zero-point path;
 *   2.C  data blocks are padded to 128-byte boundaries and the 3-bit codes are
 *        kept as three 1-bit arrays.
 * Section 1 (problem statement) motivates the shape of the interface: general
 * GPU compressors lose on launch overhead, so a whole set of messages is coded
 * in one launch (the *_batch calls), and section 3 (contributions) describes a
 * drop-in library, so every stream is self-describing.
 *
 * Compressed stream (little-endian; every section starts on a 128-byte
 * boundary of the stream; every pad byte is zero):
 *   offset 0        header, 128 B:
 *                     u32 magic 0x3143435A ("ZCC1") | u16 version 1 | u16 128
 *                     u64 n | u32 group elements 4096 | u32 NG = ceil(n/4096)
 *                     u8 exps[7] | u8 mode (0 coded, 1 raw) | u64 E (zero-point count)
 *                     u64 total_bytes | 80 zero bytes
 *   128             SM: n bytes, byte i = sign(x_i) << 7 | mantissa(x_i)
 *   off_p0          plane 0: ceil(n/64) little-endian u64 words; bit (i mod 64)
 *                   of word i/64 is bit 0 of the code of element i
 *   off_p1, off_p2  planes 1 and 2, same shape, bits 1 and 2 of the codes
 *   off_tab         NG+1 u32: entry g = zero-point values before element 4096 g
 *   off_zp          E bytes: the exponent of every element coded 000, in order
 *   with  A(x) = x rounded up to 128, W = ceil(n/64),
 *         off_p0 = A(128+n), off_p1 = off_p0 + A(8W), off_p2 = off_p1 + A(8W),
 *         off_tab = off_p2 + A(8W), off_zp = off_tab + A(4(NG+1)),
 *         total_bytes = off_zp + E.
 * Code k (1..7) stands for exps[k-1]; exps is strictly ascending.
 * Raw fallback (mode 1, only when the plan asks for it with
 * ZC_PLAN_RAW_FALLBACK): the pages describe none, but a value on the
 * zero-point path costs 19 bits, so a tensor with many of them codes to more
 * than its 16 bits per value.  When off_zp + E > 128 + 2n the stream is the
 * same header with mode 1 and total_bytes = 128 + 2n, followed by the n input
 * values unchanged (exps and E then describe the coded form that was not
 * kept); a tie keeps the coded form.  The stream is a pure function of
 * (input bits, plan): it does not depend on launch geometry, device, stream
 * or batching.
 *
 * Conventions for every call:
 *   - all buffers belong to the caller; the library never allocates, frees or
 *     synchronizes, and keeps no state between calls (the one exception is the
 *     static device workspace of zc_exponent_histogram_noalloc);
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream); device
 *     work is enqueued on it and the call returns without waiting;
 *   - "device" pointers are HIP device memory of the current device;
 *   - inputs and outputs must not overlap;
 *   - host-detectable errors return a status before anything is enqueued and
 *     nothing is written; ZC_ERR_HIP reports a failed launch;
 *   - device work is kernel launches only (no memset, copy or allocation), so
 *     every call may be captured into a HIP graph and the graph replayed with
 *     new data in the same buffers (see zc_compress for its scratch).
 */
#ifndef ZC_H
#define ZC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum zc_status {
    ZC_OK = 0,
    ZC_ERR_INVALID_ARG = 1, /* NULL pointer, bad plan, bad sigma, n > 2^32-1, k out of range */
    ZC_ERR_CAPACITY = 2,    /* an output or workspace capacity below what the call needs */
    ZC_ERR_MISALIGNED = 3,  /* BF16 buffers need 16-byte, stream buffers 128-byte alignment */
    ZC_ERR_CORRUPT = 4,     /* a stream failed validation (device-side, via the status word) */
    ZC_ERR_HIP = 5          /* the HIP runtime refused a launch */
} zc_status;

/* The exponent table ("codebook" of section 2.A): code k <-> exps[k-1].
 * exps must be strictly ascending (7 distinct values, any of 0..255);
 * flags is 0 or ZC_PLAN_RAW_FALLBACK (store the stream raw when coding would
 * make it larger, see the stream format above). */
typedef struct zc_plan {
    uint8_t exps[7];
    uint8_t flags;
} zc_plan;

#define ZC_PLAN_RAW_FALLBACK 1u

/* Section 2.A: the table from sigma alone.  For X ~ N(0, sigma^2) the
 * probability of exponent field e is P(2^(e-127) <= |X| < 2^(e-126)) for
 * e = 1..254, P(|X| < 2^-126) for e = 0 (zero and subnormals) and 0 for
 * e = 255; the 7 largest (ties to the smaller e) are returned ascending.
 * Host only, pure, thread-safe.  sigma must be finite and > 0, out non-NULL,
 * else ZC_ERR_INVALID_ARG. */
zc_status zc_plan_from_sigma(double sigma, zc_plan *out);

/* The largest stream of n elements (every element on the zero-point path,
 * section 2.B; the raw fallback form is smaller), rounded up to 128 bytes:
 * about 2.375 n + 512 bytes.  An output buffer of this capacity holds any
 * stream when the encoder's scratch sits in a workspace (zc_compress_ws,
 * zc_compress_batch_ws).  Returns 0 for n > 2^32-1. */
uint64_t zc_max_compressed_bytes(uint64_t n);

/* Encoder scratch for one tensor of n elements (a multiple of 256 bytes, a
 * little over n bytes: a staging slot of 8192 bytes per 8192 elements for
 * zero-point bytes, and the cross-workgroup words).  zc_compress and
 * zc_compress_batch keep it in the output buffer behind the largest stream;
 * the _ws calls take it from a workspace, which a caller can reuse from call
 * to call (a send buffer then needs only zc_max_compressed_bytes(n)).
 * Returns 0 for n > 2^32-1. */
uint64_t zc_compress_workspace_bytes(uint64_t n);

/* Section 2.B, compress one BF16 tensor.
 *   d_in          device, n BF16 values (raw 16-bit patterns), 16-byte aligned
 *   n             element count, 0 .. 2^32-1
 *   plan          host pointer to the exponent table
 *   d_out         device, 128-byte aligned, out_capacity bytes; receives the
 *                 stream in [0, total_bytes); [total_bytes, out_capacity) has
 *                 unspecified contents afterwards (the encoder's scratch sits
 *                 at zc_max_compressed_bytes(n))
 *   out_capacity  must be >= zc_max_compressed_bytes(n) +
 *                 zc_compress_workspace_bytes(n)
 *   d_out_bytes   device u64 (nullable): receives total_bytes
 *   stream        hipStream_t
 * Errors: ZC_ERR_INVALID_ARG, ZC_ERR_MISALIGNED, ZC_ERR_CAPACITY, ZC_ERR_HIP.
 * The stream size is also in header bytes 40..47 once the work completes.
 * With ZC_PLAN_RAW_FALLBACK the call makes two launches on the stream.  The
 * first guesses, from a sample of the input, whether the stream will come out
 * raw and writes the raw payload or the coded sections accordingly; the exact
 * rule then decides, and the second launch completes a wrong guess (it copies
 * the payload, or codes the stream).  The stream does not depend on the
 * guess.  Until the second launch has run, the header may be invalid.
 * Given-up call: workgroups of the launch wait for words that earlier
 * workgroups of the same launch write, each wait bounded (about a second).
 * With workgroups dispatched in index order no wait runs out.  Should one run
 * out anyway, its workgroup marks the segment in the scratch, the workgroup
 * that writes the header reads the mark once its own waits have passed, and
 * the call still ends; ZC_OK has already been returned, but the stream's
 * header has a zero magic (every decoder rejects it with
 * ZC_ERR_CORRUPT) and *d_out_bytes reads 0: a caller that sends
 * *d_out_bytes bytes sends nothing, and a caller that reads the header sees
 * an invalid stream.  Neither outcome passes for a valid stream.
 * HIP graphs: the call may be captured into a graph and the graph replayed
 * with new inputs in the same buffers; every replay produces the stream of
 * its input.  (The workgroups' words carry a token that mixes the call's
 * token with an 8-byte counter in the scratch, which every call advances, so
 * a replay, whose arguments repeat the captured ones, never takes the words
 * of an earlier replay for its own.)  After a given-up call, zero the scratch
 * (the workspace, or d_out past zc_max_compressed_bytes(n)) before a graph
 * that uses it is replayed. */
zc_status zc_compress(const void *d_in, uint64_t n, const zc_plan *plan, void *d_out,
                      uint64_t out_capacity, uint64_t *d_out_bytes, void *stream);

/* zc_compress with the encoder's scratch in a workspace: out_capacity need
 * only be >= zc_max_compressed_bytes(n), and nothing of d_out past the stream
 * is written.
 *   d_workspace      device, 256-byte aligned, workspace_bytes bytes, contents
 *                    arbitrary before and unspecified after the call; it may
 *                    be reused by any later call on the same stream (calls on
 *                    other streams need their own)
 *   workspace_bytes  must be >= zc_compress_workspace_bytes(n)
 * Errors as zc_compress; ZC_ERR_INVALID_ARG also for a null workspace. */
zc_status zc_compress_ws(const void *d_in, uint64_t n, const zc_plan *plan, void *d_out,
                         uint64_t out_capacity, uint64_t *d_out_bytes, void *d_workspace,
                         uint64_t workspace_bytes, void *stream);

/* Inverse of zc_compress.
 *   d_in      device, 128-byte aligned, the stream, coded or raw (in_bytes
 *             readable bytes)
 *   in_bytes  bytes available at d_in (>= total_bytes of the stream; below
 *             both off_zp of n values and 128 + 2n, ZC_ERR_CORRUPT is returned)
 *   n         the element count the caller expects
 *   d_out     device, 16-byte aligned, n BF16 values
 *   d_status  device int32 (nullable): set to 0 on success or ZC_ERR_CORRUPT.
 *             A bad header (magic, version, n, group size, exps not ascending,
 *             E > n, total_bytes inconsistent with n and E or > in_bytes) is
 *             seen by every workgroup and leaves d_out untouched.  A table or
 *             plane inconsistency is caught per 8192-element tile: the status
 *             is set, reads stay inside the stream and the affected tile's
 *             output is unspecified.
 * Errors returned: ZC_ERR_INVALID_ARG, ZC_ERR_MISALIGNED, ZC_ERR_HIP. */
zc_status zc_decompress(const void *d_in, uint64_t in_bytes, uint64_t n, void *d_out,
                        int32_t *d_status, void *stream);

/* Section 2.D, the local reduction of a reduce-scatter that runs as a zipped
 * all-to-all: each of the k streams (k = 0..ZC_MAX_BATCH) holds one peer's BF16
 * contribution to the same n elements, compressed by zc_compress; d_local is
 * the receiver's own contribution, uncompressed.  For every element i,
 * d_out[i] = BF16 of the float32 sum of d_local[i] (when given) and the k
 * decoded values, added in that order, each addition rounded to nearest (the
 * first term enters exactly), the sum rounded to BF16 nearest with ties to
 * even; a NaN sum gives 0x7FC0.  The result is a pure function of the inputs.
 *   d_streams, in_bytes  host arrays of k device stream pointers (128-byte
 *                        aligned) and the bytes readable at each
 *   k                    0..ZC_MAX_BATCH; 0 needs d_local (it then rounds it)
 *   n                    element count, 0 .. 2^32-1, the same for every stream
 *   d_local              device, n BF16 values, 16-byte aligned, nullable
 *   d_out                device, n BF16 values, 16-byte aligned; may be d_local
 *                        itself (accumulate in place), no other overlap
 *   d_status             device int32 (nullable): 0, or ZC_ERR_CORRUPT when a
 *                        stream fails validation.  A bad header in any stream
 *                        leaves d_out untouched; a table or plane inconsistency
 *                        is caught per 4096-element group (one table entry),
 *                        whose output is then unspecified (reads stay inside
 *                        every stream).
 * Errors returned: ZC_ERR_INVALID_ARG, ZC_ERR_MISALIGNED, ZC_ERR_CORRUPT (a
 * stream shorter than any stream of n values can be), ZC_ERR_HIP. */
zc_status zc_decompress_reduce(const void *const *d_streams, const uint64_t *in_bytes, uint32_t k, uint64_t n,
                               const void *d_local, void *d_out, int32_t *d_status, void *stream);

/* The online statistics that section 2.A replaces by its sigma-derived table,
 * for comparison with it and for callers with no trusted sigma.  Both calls
 * read the n BF16 values once and use a caller-owned device workspace of
 * zc_stats_workspace_bytes(n) bytes (16-byte aligned; contents unspecified
 * afterwards; two calls in flight at once need two workspaces).  Errors
 * returned: ZC_ERR_INVALID_ARG (NULL output or workspace, NULL d_in with
 * n > 0, n > 2^32-1), ZC_ERR_MISALIGNED (d_in or workspace not 16-byte,
 * outputs not 8-byte aligned), ZC_ERR_CAPACITY (workspace too small),
 * ZC_ERR_HIP. */
uint64_t zc_stats_workspace_bytes(uint64_t n);

/* d_hist (device, 256 u64) receives, for e = 0..255, the number of the n BF16
 * values whose exponent field (bits 14..7) is e.  Exact for every n. */
zc_status zc_exponent_histogram(const void *d_in, uint64_t n, void *d_workspace, uint64_t workspace_bytes,
                                uint64_t *d_hist, void *stream);

/* zc_exponent_histogram for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops or harnesses that forbid hipMalloc):
 * the same two launches and the same result, with the workspace held by the
 * library in a static device array of zc_stats_workspace_bytes() bytes
 * (512 KiB), one per GPU, kept until the process ends.  It calls no hipMalloc,
 * hipFree or other allocating routine.  All calls on one GPU share that array:
 * calls whose work overlaps on one GPU (several streams, several host
 * threads) race and must be serialized by the caller; calls in one stream are
 * ordered by it.  The array needs no clearing between calls.
 *   d_in    device, n BF16 values, 16-byte aligned (n = 0 .. 2^32-1)
 *   d_hist  device, 256 u64, 8-byte aligned
 * Errors returned: ZC_ERR_INVALID_ARG (NULL d_hist, NULL d_in with n > 0,
 * n > 2^32-1), ZC_ERR_MISALIGNED, ZC_ERR_HIP (a failed launch, or the address
 * of the array could not be obtained on the current device). */
zc_status zc_exponent_histogram_noalloc(const void *d_in, uint64_t n, uint64_t *d_hist, void *stream);

/* The table of the seven largest counts of a 256-entry histogram (host
 * array), ascending; equal counts go to the smaller field, so a histogram with
 * fewer than seven non-zero fields is filled up with the smallest unused
 * fields.  Host only, pure.  NULL hist or out gives ZC_ERR_INVALID_ARG. */
zc_status zc_plan_from_histogram(const uint64_t *hist, zc_plan *out);

/* Sigma for zc_plan_from_sigma: the root mean square of the finite values
 * (exponent field below 255; zeros count), sqrt(sum x^2 / m), which is the
 * maximum-likelihood sigma of the zero-mean Gaussian of section 2.A; 0 when no
 * value is finite.  The squares are exact in float64 and are summed in float64
 * in an order fixed by n alone (per-thread sums over a fixed grid, then fixed
 * trees), so the result is reproducible and within (m + 1024) * 2^-53 relative
 * of the exact root mean square.
 *   d_sigma   device double, receives sigma
 *   d_finite  device u64 (nullable), receives m, the count of finite values */
zc_status zc_estimate_sigma(const void *d_in, uint64_t n, void *d_workspace, uint64_t workspace_bytes,
                            double *d_sigma, uint64_t *d_finite, void *stream);

/* One message of a batched call.  Field meanings as in zc_compress. */
typedef struct zc_enc_seg {
    const void *in;
    uint64_t n;
    zc_plan plan;
    void *out;
    uint64_t out_capacity;
    uint64_t *out_bytes; /* device, nullable */
} zc_enc_seg;

/* Field meanings as in zc_decompress. */
typedef struct zc_dec_seg {
    const void *in;
    uint64_t in_bytes;
    uint64_t n;
    void *out;
    int32_t *status; /* device, nullable */
} zc_dec_seg;

#define ZC_MAX_BATCH 64

/* Compress k (1..ZC_MAX_BATCH) independent tensors in one launch, each with its
 * own plan and output buffer (per-layer gradient segments, per-destination
 * all-to-all segments); a second launch follows, over the segments whose plan
 * has ZC_PLAN_RAW_FALLBACK, when there are any.  Each output equals what
 * zc_compress gives for that segment alone (the given-up outcome of
 * zc_compress included, per segment; graph capture as for zc_compress).  segs
 * is a host array read before the call returns. */
zc_status zc_compress_batch(const zc_enc_seg *segs, uint32_t k, void *stream);

/* zc_compress_batch with every segment's scratch in one workspace (segment
 * i's at the sum of zc_compress_workspace_bytes over the segments before it):
 * each out_capacity need only be >= zc_max_compressed_bytes(n), and
 * workspace_bytes must be >= the sum over all segments.  Workspace rules as
 * for zc_compress_ws. */
zc_status zc_compress_batch_ws(const zc_enc_seg *segs, uint32_t k, void *d_workspace, uint64_t workspace_bytes,
                               void *stream);

/* Decompress k (1..ZC_MAX_BATCH) streams in one launch. */
zc_status zc_decompress_batch(const zc_dec_seg *segs, uint32_t k, void *stream);

/* Host-side view of a stream header (first 128 bytes copied to the host). */
typedef struct zc_stream_info {
    uint64_t n;
    uint64_t zero_points; /* E (of the coded form, also for a raw stream) */
    uint64_t total_bytes;
    uint32_t groups;
    zc_plan plan;         /* flags is 0 */
    uint32_t raw;         /* 1 for the raw fallback form */
} zc_stream_info;

/* Validate and unpack a header held in host memory (len >= 128).
 * Returns ZC_ERR_CORRUPT for a header the decoder would reject. */
zc_status zc_read_header(const void *host_header, uint64_t len, zc_stream_info *out);

/* Static, human-readable name of a status code. */
const char *zc_status_string(zc_status status);

#ifdef __cplusplus
}
#endif

#endif /* ZC_H */
