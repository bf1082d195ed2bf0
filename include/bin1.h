/*
 * bin1.h -- C ABI of libbin1: 1-bit sign-packed GEMV / GEMM and XOR row patching
 * on AMD Instinct MI355X (gfx950).
 *
 * The method (sources are the pages listed here by title and section):
 *  - Weight format: every weight is a sign in {-1,+1} held in one bit, and each run
 *    of 128 consecutive weights along K shares one fp16 scale, w = s_g * b, i.e.
 *    1 + 16/128 = 1.125 bits per weight.  ["Bonsai 27B: ... (feat. PrismML)",
 *    discuss.pytorch.kr, section "Binary weight format" (이진(Binary) 가중치 형식),
 *    eq. b_eff]
 *  - Kernel semantics: the packed codes are consumed directly; the sign codes are
 *    decoded and the group scale applied inside the fused product, with no dense
 *    fp16 copy of the weights, and activations/accumulation kept in high precision.
 *    [same page, section "Low-bit kernels for hybrid attention"
 *    (하이브리드 어텐션을 위한 저비트 커널)]
 *  - With +-1 weights the products are additions and subtractions and the matmul
 *    becomes bit operations.  ["PrismML Bonsai -- 1.15GB ...", jangwook.net,
 *    section "What 1-bit is" (1-bit이 뭔지부터)]
 *  - Patch: a list of rows (of a given projection in a given layer) whose bits are
 *    flipped in place; it adds no matmul at inference and the same XOR removes it.
 *    It is defined only for true binary weights (for ternary codes an XOR can leave
 *    the valid states).  ["LocalLLaMA ... XOR patch 'Bankai'", insights.marvin-42.com,
 *    sections "Key points" and "Why it holds only for true 1-bit models"]
 *
 * Layouts (row-major, contiguous, little-endian).  K is the input width, N the number
 * of output rows, M the number of activation rows (tokens):
 *   x       fp16   [M][K]
 *   Wbits   uint32 [N][K/32]  weight (n, k) is bit (k % 32) of word [n][k / 32];
 *                             bit 1 means +1, bit 0 means -1 (LSB-first along K)
 *   scales  fp16   [N][K/128] scale of weights k in [128g, 128g+128) of row n
 *   y       fp16   [M][N]     y[m][n] = sum_k scales[n][k/128] * w(n,k) * x[m][k],
 *                             accumulated in fp32, rounded once to fp16 (nearest-even)
 *   Abits   uint32 [M][K/32]  +-1 activations packed like Wbits (popcount mode)
 *
 * Conventions for every call:
 *  - Data pointers are DEVICE pointers on the current HIP device, owned by the caller.
 *    The library never allocates, frees or synchronises; a call validates its
 *    arguments on the host and then only enqueues kernels on `stream` (a hipStream_t
 *    passed as void*; NULL means the legacy default stream).  Calls may therefore be
 *    captured into a HIP graph.
 *  - Validation happens before anything is enqueued; on any error nothing is enqueued
 *    and the outputs are untouched.
 *  - Requirements: M >= 0, N >= 0, K >= 128, K % 128 == 0; x, Wbits, scales, y, Abits
 *    16-byte aligned; y must not overlap any input.  Products also need N < 2^24 - 64
 *    and x, Wbits and y each under 2 GiB (else BIN1_ERR_SHAPE).  A product with no
 *    outputs (M == 0 or N == 0) returns BIN1_OK without enqueuing anything; its
 *    pointers are not read and may be NULL.  (K cannot be 0: a row is a whole number of
 *    128-weight groups, each with its scale.)
 *  - Device-side faults surface at the caller's next synchronisation, as with any
 *    HIP kernel.  BIN1_ERR_LAUNCH carries the HIP error text in bin1_last_error().
 *  - The library is stateless apart from a thread-local error string: calls are
 *    reentrant and may run concurrently on different streams.
 */
#ifndef BIN1_H
#define BIN1_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BIN1_ABI_VERSION 1

typedef enum bin1_status {
    BIN1_OK = 0,
    BIN1_ERR_NULL = -1,     /* a required pointer is NULL                               */
    BIN1_ERR_SHAPE = -2,    /* M, N, K (or a count) out of range / K not a multiple of 128 */
    BIN1_ERR_ALIGN = -3,    /* a data pointer is not 16-byte aligned                     */
    BIN1_ERR_ALIAS = -4,    /* the output range overlaps an input range                  */
    BIN1_ERR_DEVICE = -5,   /* a pointer is not device memory of the current device      */
    BIN1_ERR_LAUNCH = -6    /* the HIP runtime refused the launch (see bin1_last_error)  */
} bin1_status;

/* Decode GEMV / small-batch product: y = x * W^T with W = scales (x) signs, per the
 * layouts above.  Tuned for M in 1..16; correct for any M >= 1 (M > 16 is routed to
 * the prefill kernel).  The signs are expanded without multiplies and the group scale
 * is applied once per 128-weight group; accumulation is fp32; y is fully overwritten. */
int bin1_gemv(const void *x, const uint32_t *Wbits, const void *scales, void *y,
              int M, int K, int N, void *stream);

/* Same-input fusion: `count` (1..4) products that read the same activations x [M][K]
 * (such as the q/k/v or gate/up projections of one layer), enqueued as one launch when
 * M <= 16.  Wbits, scales, y and N are HOST arrays of `count` entries; entry i describes
 * matrix i exactly as in bin1_gemv (Wbits[i] [N[i]][K/32], scales[i] [N[i]][K/128],
 * y[i] [M][N[i]]).  Every y[i] must be disjoint from every input and from the other
 * outputs.  Results equal `count` separate bin1_gemv calls; a matrix with N[i] == 0 is
 * skipped.  At M == 1, matrices stored back to back (weights, scales and outputs of one
 * each starting where the previous one's end, as in a fused q/k/v allocation) are run as
 * one taller matrix, which launches faster and gives the same results. */
int bin1_gemv_group(const void *x, int count, const uint32_t *const *Wbits,
                    const void *const *scales, void *const *y, const int *N,
                    int M, int K, void *stream);

/* The product of bin1_gemv with a caller-owned scratch area, which lets long small-batch products
 * split K over workgroups.  With 2 <= M <= 16 tokens every workgroup must bring the activations of
 * its K range into on-chip memory, and for K > 4096 that dwarfs its share of the weights; with
 * the workspace each workgroup stages one 4096-wide chunk of x for more rows, stores fp32 partial
 * sums per chunk in the workspace, and a second kernel adds the chunks in a fixed order (chunk 0,
 * 1, ...) and rounds once to fp16.  Decode speed is bounded by bandwidth over weight bytes
 * ["Bonsai 27B" page, section "Low-bit kernels for hybrid attention"]; this keeps the per-CU
 * activation stream below the weight stream.
 * workspace: device memory, 256-byte aligned, at least bin1_gemv_workspace_bytes(M, K, N) bytes,
 * not overlapping x, Wbits, scales or y; it holds nothing between calls (no clearing needed), but
 * two calls in flight at once must not share it.  When that size is 0 (the shape takes no split
 * path) workspace may be NULL and the call is bin1_gemv.  Results equal bin1_gemv's within the
 * parity bar (the summation order differs); errors as bin1_gemv, plus BIN1_ERR_NULL / _SHAPE /
 * _ALIGN / _ALIAS for a missing, short, misaligned or overlapping workspace. */
size_t bin1_gemv_workspace_bytes(int M, int K, int N);
int bin1_gemv_ws(const void *x, const uint32_t *Wbits, const void *scales, void *y, int M, int K, int N,
                 void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): bin1_gemv_ws with the library's own scratch instead of
 * a caller's workspace.  The scratch is a static device array of 4 MiB that every GPU the library
 * runs on holds until the process ends; its device address is looked up on the first call on each
 * device (so make that first call outside a capture).  Shapes whose workspace
 * (bin1_gemv_workspace_bytes) exceeds 4 MiB return BIN1_ERR_SHAPE before anything is enqueued.
 * All calls on one GPU share that GPU's array: calls that overlap in time on one GPU (on different
 * streams without ordering between them) race; calls ordered on one stream do not.  Nothing has to
 * be cleared between calls.  Results are bit-identical to bin1_gemv_ws on the same inputs. */
int bin1_gemv_noalloc(const void *x, const uint32_t *Wbits, const void *scales, void *y, int M, int K, int N,
                      void *stream);

/* Prefill product, same arguments and result as bin1_gemv; tuned for M >= 256 (the
 * pages note that prompt processing is compute-bound: ["Bonsai 27B", section "Low-bit
 * kernels for hybrid attention"]).  The sign bits are expanded in registers into fp16 +-|scale|
 * matrix-core operands (activations staged through LDS) and contracted with fp32
 * accumulation.  Correct for any M >= 1. */
int bin1_gemm_prefill(const void *x, const uint32_t *Wbits, const void *scales, void *y,
                      int M, int K, int N, void *stream);

/* Ternary g128 products ["Bonsai 27B", section on the ternary weight format: each weight
 * t in {-1, 0, +1}, w = s_g * t, one fp16 scale per group of 128; its deployment section:
 * current kernels keep each ternary value in a 2-bit slot]:
 *   y[m][n] = sum_k s[n][k/128] * t(n,k) * x[m][k]
 *   Tbits  uint32 [N][K/16]: weight k of row n is the 2-bit slot at bits 2(k%16), 2(k%16)+1
 *          of word [n][k/16] (LSB first); low bit = nonzero, high bit = negative: 00 -> 0,
 *          01 -> +1, 11 -> -1, and 10 reads as 0.
 * Everything else (x, scales, y, requirements, errors, streams) is as for bin1_gemv and
 * bin1_gemm_prefill.  bin1_gemv_t2 runs M == 1 on the block-scaled matrix cores and other M
 * on the prefill kernel; bin1_gemm_prefill_t2 is tuned for M >= 256.  There is no XOR patch
 * for ternary weights (the Bankai page: XOR patches need true binary codes). */
int bin1_gemv_t2(const void *x, const uint32_t *Tbits, const void *scales, void *y,
                 int M, int K, int N, void *stream);
int bin1_gemm_prefill_t2(const void *x, const uint32_t *Tbits, const void *scales, void *y,
                         int M, int K, int N, void *stream);
/* Same-input fusion for ternary weights: as bin1_gemv_group, with Tbits[i] [N[i]][K/16];
 * one launch when M == 1. */
int bin1_gemv_group_t2(const void *x, int count, const uint32_t *const *Tbits,
                       const void *const *scales, void *const *y, const int *N,
                       int M, int K, void *stream);

/* +-1 activations times +-1 weights, exact:
 *   y[m][n] = sum_k a(m,k) * w(n,k) = K - 2 * popcount(Abits[m] xor Wbits[n])  (int32).
 * Scales are not used.  ["PrismML Bonsai -- 1.15GB ...", section "What 1-bit is"] */
int bin1_gemv_pm1(const uint32_t *Abits, const uint32_t *Wbits, int32_t *y,
                  int M, int K, int N, void *stream);

/* XOR row patch, in place: for each entry r of rowlist (device int32[nrows]) every
 * word of row r of Wbits ([N][K/32]) is complemented, i.e. all K signs of output row
 * r are flipped (y[:, r] -> -y[:, r]); scales are untouched.  Calling it again with
 * the same list removes the patch.  The complement is applied as atomic XORs, so entries
 * commute: a row listed an even number of times in one call ends unchanged, an odd number
 * of times complemented (a patch's rows are normally distinct; repeats are well defined,
 * not an error).  Entries outside [0, N) are skipped and, if bad_rows (device int32*,
 * may be NULL) is given, counted into *bad_rows by atomic add (the caller zeroes it).
 * nrows == 0 is a no-op.  Order the call on the same stream as the products that
 * read Wbits.  ["LocalLLaMA ... XOR patch 'Bankai'", section "Key points"] */
int bin1_xor_patch_apply(uint32_t *Wbits, const int32_t *rowlist, int nrows,
                         int K, int N, int32_t *bad_rows, void *stream);

/* The same patch over many matrices in one launch -- (layer, projection, row) records.
 * Wtab (device uint32_t*[nmat]), Ktab and Ntab (device int32[nmat]) describe the
 * matrices; entries (device int32[nentries][2]) holds (matrix id, row) pairs.  Entries
 * with a matrix id outside [0, nmat), a row outside [0, N_id), or a K_id that is not a
 * positive multiple of 128 are skipped and counted into *bad_rows when given.  As for the
 * single-matrix call, repeated entries commute (an even count leaves the row unchanged).
 * nentries == 0 is a no-op. */
int bin1_xor_patch_apply_multi(uint32_t *const *Wtab, const int32_t *Ktab, const int32_t *Ntab,
                               int nmat, const int32_t *entries, int nentries,
                               int32_t *bad_rows, void *stream);

/* Bit-granular XOR patch over many matrices in one launch ["LocalLLaMA ... XOR patch
 * 'Bankai'", experiments section: random flips of single bits of the MLP weights, e.g.
 * 500K of them].  Wtab, Ktab, Ntab describe the matrices as in bin1_xor_patch_apply_multi;
 * entries (device int32[nentries][3]) holds (matrix id, row, k) records, each flipping the
 * sign bit of weight k of that row (y[:, row] changes by -2 s w x_k).  Records may repeat:
 * flips are atomic XORs, so the result is independent of order, a bit listed an even number
 * of times is unchanged, and the same list applied again removes the patch.  Records with a
 * matrix id outside [0, nmat), a row outside [0, N_id), k outside [0, K_id), a K_id that is
 * not a positive multiple of 128, or a misaligned matrix are skipped and counted into *bad
 * (device int32*, may be NULL; the caller zeroes it).  nentries == 0 is a no-op.  Order it
 * on the stream of the products that read the weights. */
int bin1_xor_bits_apply(uint32_t *const *Wtab, const int32_t *Ktab, const int32_t *Ntab, int nmat,
                        const int32_t *entries, int nentries, int32_t *bad, void *stream);

/* Scale ranking of rows, the mechanics of targeting patches by scale factors [same page,
 * experiments section].  scales: device fp16 [N][K/128] (16-byte aligned).  Writes
 * score (device int64[N]): the sum over the row's groups of |scale|, exactly, in units of
 * 2^-24 (an inf/NaN scale counts as its magnitude bits would, (f + 2^10) << 30), and order
 * (device int32[N]): the rows by score, largest first, equal scores by ascending row.
 * Requires 0 <= N <= 2^20 (the ranking counts over all pairs; N == 0 is a no-op), K >= 128,
 * K % 128 == 0, and no overlap between scales, score and order. */
int bin1_rank_rows_by_scale(const void *scales, int N, int K, int64_t *score, int32_t *order, void *stream);

/* ------------------------------------------------------------------------------------
 * Decode-step chain: a sequence of dependent stages in ONE persistent launch.
 * Stage s = `count` (1..4) products that read the same activations x_s (fp16 [K_s]), M = 1;
 * stage s+1 starts only after every output of stage s is written (the batch-1 decode order:
 * q/k/v, o, gate/up, down per layer, then lm_head).  Launch and synchronisation latency, not
 * weight bandwidth, bound batch-1 decode on datacenter GPUs ["Bonsai 27B" page, section
 * "Low-bit kernels for hybrid attention"]; the chain keeps one workgroup per CU resident for
 * the whole step, streams the next stage's weights while a stage waits, and orders stages
 * with device-scope release/acquire flags in the workspace.
 * Requirements: K_s % 256 == 0 and K_s <= 20480, every N >= 1; the GPU has at least 256
 * compute units; the products follow bin1_gemv's layouts.  An output may be (and usually is) a later stage's x, but
 * must not overlap its own stage's x, any Wbits or scales of the chain, or another output of
 * its stage.
 * The workspace (device memory, caller-owned, bin1_chain_workspace_bytes(nstages) bytes,
 * 256-byte aligned) holds the stage table, the flags and a run counter; it must not be shared
 * by two chains running at the same time.  Runs never need it cleared again (flags only
 * grow), so one prepared chain can be captured into a HIP graph and replayed.  A stage wait
 * is bounded (about seconds); if it gives up, that run's results are invalid and
 * bin1_chain_status reports it (the flag stays set until the chain is prepared again).  */
typedef struct bin1_stage {
    const void *x;                 /* device fp16 [K] */
    int K;
    int count;                     /* 1..4 */
    const uint32_t *Wbits[4];      /* device, [N[i]][K/32] */
    const void *scales[4];         /* device fp16 [N[i]][K/128] */
    void *y[4];                    /* device fp16 [N[i]] */
    int N[4];
} bin1_stage;

typedef struct bin1_chain_plan {   /* filled by bin1_chain_prepare; plain host struct */
    void *workspace;
    int nstages;
    int spmax;                     /* ceil(max_s ceil(K_s / 1024) / 4): selects the kernel variant */
    int max_tiles;                 /* most row tiles one workgroup owns in any stage */
    int spin_limit;                /* polls per stage wait before giving up; 0 (set by prepare) =
                                      the default of about seconds; the caller may lower it */
} bin1_chain_plan;

size_t bin1_chain_workspace_bytes(int nstages);

/* Validate the stages and write the stage table into `workspace` (synchronous host->device
 * copies; not for use inside graph capture).  Fills *plan. */
int bin1_chain_prepare(const bin1_stage *stages, int nstages, void *workspace, size_t workspace_bytes,
                       bin1_chain_plan *plan);

/* Enqueue one run of a prepared chain on `stream`.  Capturable. */
int bin1_gemv_chain(const bin1_chain_plan *plan, void *stream);

/* Synchronously read the workspace: *runs = completed runs, *error = 1 if a wait gave up. */
int bin1_chain_status(const bin1_chain_plan *plan, int *runs, int *error);

/* Measurement helper (does none of the method's arithmetic): reads `bytes` of device memory at
 * buf once, with 16-byte nontemporal loads spread over `grid` workgroups of 256 threads, `unroll`
 * loads in flight per thread (4, 8 or 16), and writes one XOR digest per wave into sink (device
 * uint32 [4 * grid]).  Timing it gives the HBM read rate this GPU sustains, the reference against
 * which the decode products' bandwidth is measured (decode speed is bounded by bandwidth over weight
 * bytes: "Bonsai 27B" page, section "Low-bit kernels for hybrid attention").  Requires buf 16-byte
 * aligned, bytes a positive multiple of 16, 1 <= grid <= 65536, and sink not overlapping buf. */
int bin1_stream_read(const void *buf, size_t bytes, uint32_t *sink, int grid, int unroll, void *stream);

/* Measurement helper (does none of the method's arithmetic): `grid` workgroups of `waves` waves
 * (4: one per SIMD, or 8: two) each issue iters x 12 independent fp16 matrix-core products
 * (32 x 32 x 16, 32768 flops each) with nothing else in the loop.  Timing it gives the fp16 MFMA
 * rate this GPU sustains, the reference for the prefill product, which is compute-bound
 * ("Bonsai 27B" page, section "Low-bit kernels for hybrid attention").  The rate depends on the
 * operand values (their bit activity sets the power drawn and so the clock held), so the caller
 * supplies them: operands is device fp16 [2][64][8], lane l's A fragment (row l % 32, k = 8 (l / 32)
 * .. + 7) then its B fragment (k = 8 (l / 32) .. + 7, column l % 32).  Writes, for every wave w,
 * sink[w] = the fp32 sum over the 12 accumulators of their row-0, column-0 element, which is
 * 12 * iters * D00 (D = A B) when all partial sums are exact in fp32 (small integer operands).
 * Requires 1 <= grid <= 65536, waves 4 or 8, 1 <= iters <= 1000000, operands 16-byte aligned,
 * sink (device float [grid * waves]) 4-byte aligned and not overlapping operands. */
int bin1_mfma_rate(const void *operands, float *sink, int grid, int waves, int iters, void *stream);

/* Diagnostic: the kernel variant(s) and grid that a product call would launch for these shapes,
 * from the same dispatch code the calls run (nothing is launched; no device is needed).
 * op: 0 = bin1_gemv (count == 1) or bin1_gemv_group, 1 = bin1_gemv_t2 or bin1_gemv_group_t2,
 * 2 = bin1_gemm_prefill, 3 = bin1_gemm_prefill_t2, 4 = bin1_gemv_ws given a large enough
 * workspace (count == 1 for 2, 3 and 4).  N: host int[count],
 * the row counts as the call would launch them (matrices a group call runs as one taller matrix
 * are given as one).  Writes a NUL-terminated text such as "gemv_mx<1,1,1,0,0,4,1> grid=384" into
 * name (len bytes; launches separated by ';').  Requires M >= 1, K >= 128, K % 128 == 0 and
 * 1 <= N[i] < 2^24 - 64; BIN1_ERR_SHAPE also if len is too small. */
int bin1_kernel_variant(int op, int M, int K, int count, const int *N, char *name, int len);

/* Static description of a status code. */
const char *bin1_status_string(int status);

/* Thread-local detail of the last error returned on this thread ("" if none). */
const char *bin1_last_error(void);

/* == BIN1_ABI_VERSION */
int bin1_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BIN1_H */
