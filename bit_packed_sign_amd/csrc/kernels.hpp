// kernels.hpp -- internal launchers behind the C ABI (include/bin1.h).  Each launcher
// assumes its arguments were validated by the API layer and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace bin1 {

// Every product launcher takes an optional `desc`: when it is given, nothing is launched and the
// name of the kernel variant and its grid that the call would launch are appended to it instead
// (the library's variant query runs the same dispatch code as the launches).
//
// Up to kMaxMats products that read the same activation vector (e.g. q/k/v or gate/up),
// decoded in one launch.  tile_end[] is filled in by the launcher (cumulative row tiles).
constexpr int kMaxMats = 4;
struct MxSet {
    const uint32_t *W[kMaxMats];
    const uint16_t *S[kMaxMats];
    uint16_t *y[kMaxMats];
    int N[kMaxMats];
    int tile_end[kMaxMats];
    int count;
};

// Persistent chain of dependent decode stages (one launch for a whole decode step).
constexpr int kChainWgs = 256;                 // workgroups, one per CU of the MI355X
struct ChainHeader {
    int nstages;
    int gen;          // completed runs (only grows)
    int exit_count;   // workgroups finished, over all runs (only grows)
    int error;        // set when a stage wait gave up
    int spmax;
    int max_tiles;
    int withhold;     // fault injection for tests: nonzero = workgroup 0 never publishes stage 0,
                      // so every later wait can only end through its spin limit
    int pad[9];
};
// One stage as the kernel sees it.  Work is split into units of `rt` row tiles (16 rows each)
// of one matrix; unit_end[] is cumulative over the stage's matrices.
struct ChainStage {
    const uint16_t *x;
    const uint32_t *W[kMaxMats];
    const uint16_t *S[kMaxMats];
    uint16_t *y[kMaxMats];
    int N[kMaxMats];
    int unit_end[kMaxMats];
    int count;
    int K;
    int nunits;
    int rt;
    int x_written;    // some stage of the chain writes x: read it device-coherently
    int pad;
};
// Pairs (1024-wide K slices) each of the 4 waves takes for a stage of width K.
__host__ __device__ inline int chain_pairs_per_wave(int K) { return ((K + 1023) / 1024 + 3) / 4; }
// Row tiles per unit: the kernel's register slot holds spmax (row tile, pair) blocks.
__host__ __device__ inline int chain_unit_tiles(int spmax, int K) { return spmax / chain_pairs_per_wave(K); }
// Dynamic LDS of the chain kernel, or 0 if it does not fit in one workgroup's LDS.
size_t chain_lds_bytes(int spmax, int nstages, int max_tiles);
hipError_t launch_gemv_chain(ChainHeader *hdr, int *done, const ChainStage *table, int nst, int spmax,
                             int max_tiles, long spin_limit, hipStream_t st);

// Largest K the block-scaled decode kernel takes (longer rows use the select kernel).
int mx_max_k();
// Whether a 2 <= M <= 8 product runs as M copies of the one-token grid (launch_gemv_mx, mt = M).
bool mx_tokens_handles(int M, int K, const MxSet &set);
// mt tokens (1..8): x is [mt][K] and every y of the set [mt][N]; the one-token grid is launched
// mt times over, one copy per token.
hipError_t launch_gemv_mx(const uint16_t *x, const MxSet &set, int K, hipStream_t st, std::string *desc = nullptr,
                          int mt = 1);
// The same product for ternary weights in 2-bit slots (W pointers of the set: uint32 [N][K/16]).
hipError_t launch_gemv_mx_t2(const uint16_t *x, const MxSet &set, int K, hipStream_t st,
                             std::string *desc = nullptr, int mt = 1);

hipError_t launch_gemv(const uint16_t *x, const uint32_t *W, const uint16_t *S, uint16_t *y,
                       int M, int K, int N, hipStream_t st, std::string *desc = nullptr);
// Small-batch product (2 <= M <= 16) on fp16 MFMA with the tokens as the A rows.
// 2 <= M <= 16 tokens, 1..4 products sharing x (tile_end filled in by the launcher).
// With `part` (device scratch of smallm_split_bytes(M, K, N[0]) bytes) a one-matrix product with
// K > 4096 splits K over workgroups: fp32 partial sums per 4096-wide chunk, then a reduction.
hipError_t launch_gemv_smallm(const uint16_t *x, const MxSet &set, int M, int K, hipStream_t st,
                              std::string *desc = nullptr, float *part = nullptr);
// Scratch bytes of the split-K small-batch product (0 when the shape does not split).
size_t smallm_split_bytes(int M, int K, int N);
// y[i] = fp16(sum over chunks c of part[c][i]) in ascending c (i = m * N + n), one thread per output.
hipError_t launch_smallm_reduce(const float *part, int nchunk, int MN, uint16_t *y, hipStream_t st);
// 2 <= M <= 8 on the block-scaled matrix cores (gemv_mxm.hip): K a multiple of 1024, and K <= 4096
// unless a one-matrix product brings the split scratch.  launch_gemv_smallm routes such shapes there
// when they are tall enough to pay for the kernel's activation conversion (mxm_handles).
bool mxm_handles(int M, int K, const MxSet &set, bool have_part);
hipError_t launch_gemv_mxm(const uint16_t *x, const MxSet &set, int M, int K, hipStream_t st, std::string *desc,
                           float *part);
hipError_t launch_prefill(const uint16_t *x, const uint32_t *W, const uint16_t *S, uint16_t *y,
                          int M, int K, int N, hipStream_t st, std::string *desc = nullptr);
// Ternary weights in 2-bit slots: T uint32 [N][K/16].
hipError_t launch_prefill_t2(const uint16_t *x, const uint32_t *T, const uint16_t *S, uint16_t *y,
                             int M, int K, int N, hipStream_t st, std::string *desc = nullptr);
hipError_t launch_pm1(const uint32_t *A, const uint32_t *W, int32_t *y, int M, int K, int N,
                      hipStream_t st);
hipError_t launch_xor_bits(uint32_t *const *Wtab, const int32_t *Ktab, const int32_t *Ntab, int nmat,
                           const int32_t *entries, int n, int32_t *bad, hipStream_t st);
hipError_t launch_rank_rows(const uint16_t *S, int N, int K, int64_t *score, int32_t *order, hipStream_t st);
hipError_t launch_xor_patch(uint32_t *W, const int32_t *rows, int nrows, int K, int N,
                            int32_t *bad, hipStream_t st);
hipError_t launch_xor_patch_multi(uint32_t *const *Wtab, const int32_t *Ktab, const int32_t *Ntab,
                                  int nmat, const int32_t *entries, int nentries, int32_t *bad,
                                  hipStream_t st);

// Streaming read of `bytes` (multiple of 16) into a per-wave digest sink[4 * grid].
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, int grid, int unroll, hipStream_t st);
hipError_t launch_mfma_rate(const void *ab, float *sink, int grid, int waves, int iters, hipStream_t st);

// Shared by the entry points (defined with the C ABI's validation): the thread-local error text,
// and bin1_gemv with a scratch area for the split-K path (caller_ws: a caller's workspace, checked
// like its other pointers; otherwise the library's own static array).
int set_error(int status, const char *what);
int gemv_scratch(const char *fn, const void *x, const uint32_t *Wbits, const void *scales, void *y, int M, int K,
                 int N, void *ws, size_t ws_bytes, bool caller_ws, void *stream);

}  // namespace bin1
