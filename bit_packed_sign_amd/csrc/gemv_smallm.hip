// gemv_smallm.hip -- small-batch decode product (2 <= M <= 16 tokens) on fp16 MFMA.
//
// y[m][n] = sum_k s[n][k/128] * w(n,k) * x[m][k] ["Bonsai 27B" page, section "Binary weight
// format", eq. b_eff], fused decode with fp32 accumulation ["Bonsai 27B" page, section
// "Low-bit kernels for hybrid attention"].  With M tokens each weight serves M products, so
// the expansion of a sign costs 1/M per product.
//
// v_mfma_f32_16x16x32_f16: the tokens are the 16 A rows (x is fp16 already, so A is exact;
// rows past M are zero) and 16 weight rows are the B columns.  Lane (n, b) of a wave owns
// ONE scale group of row n -- group 4*wave + b of the current 4096-wide K chunk -- so a tile
// costs each lane one 16-byte load and one scale load, and the group scale goes straight into
// the B operand as fp16 +-|s| (a negative scale is folded into the sign bits).
//
// k order inside an MFMA: MFMA t = 4j + q of a group (word j, quarter q) covers k = 32j + 8q ..
// 32j + 8q + 7 in natural order: lane (n, b)'s B pair p holds the signs of bits 8q + 2p and
// 8q + 2p + 1 of word j -- one packed 16-bit shift of the half-word holding them (read by both
// halves) and one and-or per fp16 pair -- and its A operand is those 8 activations as stored.
//
// x goes through LDS: the workgroup copies each 4096-wide K chunk of the 16 token rows
// (128 KB) with contiguous 16-byte loads, all in flight at once; each wave then reads its A
// operands once per chunk and reuses them for every tile of the batch.
// Read straight from memory, every A load would touch 64 cache lines.  The merge table
// reuses the same LDS once the batch's last chunk is done.
#include <cstdio>
#include <string>

#include "common.hpp"
#include "kernels.hpp"

namespace bin1 {

namespace {

typedef unsigned u4v __attribute__((ext_vector_type(4)));
typedef unsigned short us2v __attribute__((ext_vector_type(2)));

constexpr int kRsrcFlags = 0x00020000;
constexpr unsigned kOob = 0x80000000u;
constexpr int kNT = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcFlags);
}

constexpr int kWaves = 8;                            // waves per workgroup
constexpr int kChunkGroups = 4 * kWaves;             // scale groups per K chunk (4096 k)
constexpr int kChunkK = 128 * kChunkGroups;
constexpr int kXRow = kChunkK + 8;                   // LDS row stride of the staged chunk (halves)
// thread t stages and wave w reads the chunk's columns [512 w, 512 w + 512): waves never share them
static_assert(kChunkK == 8 * 64 * kWaves, "one 512-column slice of the chunk per wave");
constexpr int kXBytes = 16 * kXRow * 2;              // 16 token rows
static_assert(kChunkK == 8 * 64 * kWaves && kWaves == 8, "one 16-byte load per thread per token row");

// B operand of quarter Q: pair p = (+-|s| for bit 8Q + 2p, for bit 8Q + 2p + 1) of nw, bit 1 of
// nw meaning a negative product.
template <int Q>
__device__ __forceinline__ half8 expand_q(uint32_t nw, uint32_t s2abs)
{
    const us2v v = us2v((unsigned short)(Q < 2 ? nw : nw >> 16));
    u4v d;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int bit = 8 * (Q & 1) + 2 * p;
        const us2v sh{(unsigned short)(15 - bit), (unsigned short)(14 - bit)};
        d[p] = (__builtin_bit_cast(uint32_t, v << sh) & 0x80008000u) | s2abs;
    }
    return __builtin_bit_cast(half8, d);
}

struct SmSlot {
    u4v w;          // this lane's group: 4 words of row n
    uint32_t s;     // its fp16 scale
};

struct SmTile {     // one tile of the workgroup, resolved once
    const uint32_t *W;
    const uint16_t *S;
    uint16_t *y;
    int row0, N;    // N = 0: no tile (its loads return zeros, nothing is stored)
};

// Work: workgroup g takes tiles g, g + G, ... (at most TB of them); for these it walks K in
// 4096-wide chunks.  Slot [d][t] holds tile t's group for chunk c = D*j + d, so D chunks of
// every tile are in flight; a wave's A operands are built once per chunk, and the next chunk
// of x is already loading (into registers) while the current one is used.  The waves' partial
// tiles are merged through LDS at the end.  Tile slots past the workgroup's tiles compute on
// zeros and are never stored.  D = 0 is the one-chunk case (K <= 4096): no prefetch, no
// refills.  Loads are never issued under a branch (the compiler would then wait for every
// load in flight where the paths meet).
template <int TB, int D, bool SPLIT>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemv_smallm_kernel(const uint16_t *__restrict__ x, int M, int K, int tq, int tr, int G, MxSet set,
                        float *__restrict__ part)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // staged chunk [16][kXRow]
    float *red = reinterpret_cast<float *>(xs);                     // then [tile][wave][lane][4]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, b = lane >> 4;
    const int wpr = K >> 5, spr = K >> 7;
    const int nchunk = (spr + kChunkGroups - 1) / kChunkGroups;
    // the scalars come first in the argument list and arrive preloaded in registers; the tile
    // count is split on the host (tiles = tq * G + tr, G the grid size)
    // SPLIT: workgroup b takes K chunk cw = b / G only, for tile group b % G, and stores fp32
    // partial sums of that chunk (the reduction over chunks is a second kernel)
    const int cw = SPLIT ? (int)blockIdx.x / G : 0;
    const int gid = (int)blockIdx.x - cw * G;
    const int nb = tq + (gid < tr ? 1 : 0);                                                // <= TB
    const __amdgpu_buffer_rsrc_t rx = rsrc(x, (unsigned)M * (unsigned)K * 2u);

    // thread t's share of a chunk: 8 k of every token row; rows past M are outside the buffer
    // range, and k past K starts from an out-of-range base, so both load zeros.  Register m
    // holds token row (m + rot) % 16: every workgroup reads the same activations, and starting
    // each one at a different row spreads their simultaneous requests over the L2 channels.
    u4v xr[16];
    const int rot = (int)(blockIdx.x & 15);
    auto fetch_x = [&](int c) {
        const unsigned kc = (unsigned)((c + cw) * kChunkK) + 8u * threadIdx.x;
        const unsigned base = kc < (unsigned)K ? kc * 2u : kOob;
#pragma unroll
        for (int m = 0; m < 16; ++m)
            xr[m] = __builtin_amdgcn_raw_buffer_load_b128(rx, base + (unsigned)((m + rot) & 15) * (unsigned)K * 2u, 0, 0);
    };
    fetch_x(0);                                       // first: staging it waits on nothing else
    __builtin_amdgcn_sched_barrier(0);               // (ahead of the argument-table loads)

    // lane t resolves tile slot t (matrix, first row) with vector selects; the results are
    // then read into scalar registers, so every wave holds them at the cost of a few readlanes
    SmTile tl[TB];
    {
        const int tile = gid + lane * G;
        const int m1 = set.count > 1 && tile >= set.tile_end[0], m2 = set.count > 2 && tile >= set.tile_end[1],
                  m3 = set.count > 3 && tile >= set.tile_end[2];
        auto sel = [&](auto a0, auto a1, auto a2, auto a3) { return m3 ? a3 : m2 ? a2 : m1 ? a1 : a0; };
        const int row0 = (tile - sel(0, set.tile_end[0], set.tile_end[1], set.tile_end[2])) * 16;
        const int N = lane < nb ? sel(set.N[0], set.N[1], set.N[2], set.N[3]) : 0;
        const unsigned long long W = (unsigned long long)sel(set.W[0], set.W[1], set.W[2], set.W[3]);
        const unsigned long long S = (unsigned long long)sel(set.S[0], set.S[1], set.S[2], set.S[3]);
        const unsigned long long Y = (unsigned long long)sel(set.y[0], set.y[1], set.y[2], set.y[3]);
        auto rl = [](unsigned long long v, int t) {       // readlane gives an int: no sign extension
            const unsigned lo = (unsigned)__builtin_amdgcn_readlane((unsigned)v, t);
            const unsigned hi = (unsigned)__builtin_amdgcn_readlane((unsigned)(v >> 32), t);
            return ((unsigned long long)hi << 32) | lo;
        };
#pragma unroll
        for (int t = 0; t < TB; ++t)
            tl[t] = SmTile{reinterpret_cast<const uint32_t *>(rl(W, t)), reinterpret_cast<const uint16_t *>(rl(S, t)),
                           reinterpret_cast<uint16_t *>(rl(Y, t)), __builtin_amdgcn_readlane(row0, t),
                           __builtin_amdgcn_readlane(N, t)};
    }
    constexpr int DS = D > 0 ? D : 1;
    SmSlot ring[DS][TB];
    // No selects here (the compiler turns them into branches that wait on loads in flight):
    // rows at or past N fall outside the buffer range and load zeros, and a group past K (or a
    // refill past the last chunk) reloads the row's last group, which meets x = 0.
    auto issue = [&](const SmTile &T, int c, SmSlot &sl) {
        const unsigned row = (unsigned)(T.row0 + n);
        const unsigned gb = (unsigned)min((c + cw) * kChunkGroups + 4 * wave + b, spr - 1);
        const unsigned live = c + cw < nchunk ? (unsigned)T.N : 0u;  // past the last chunk: no range
        const __amdgpu_buffer_rsrc_t rW = rsrc(T.W, live * (unsigned)wpr * 4u);
        const __amdgpu_buffer_rsrc_t rS = rsrc(T.S, live * (unsigned)spr * 2u);
        // mul24 row products (rows < 2^24) keep the wait counts exact
        sl.w = __builtin_amdgcn_raw_buffer_load_b128(rW, (mul24(row, (unsigned)wpr) + 4u * gb) * 4u, 0, kNT);
        sl.s = __builtin_amdgcn_raw_buffer_load_b16(rS, (mul24(row, (unsigned)spr) + gb) * 2u, 0, 0);
    };
#pragma unroll
    for (int d = 0; d < DS; ++d)
#pragma unroll
        for (int t = 0; t < TB; ++t) issue(tl[t], d, ring[d][t]);

    float4v acc[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] = float4v{0.f, 0.f, 0.f, 0.f};
    // stage chunk c's x (in xr) into LDS and start loading chunk c + 1 (past K: zeros, no
    // traffic).  Staging comes last in a chunk, so its wait is for loads issued before that
    // chunk's refills.  Wave w stages columns [512 w, 512 w + 512) of every token row, and its A
    // operands come from those same columns: no other wave reads them, and one wave's LDS
    // accesses execute in order, so no workgroup barrier is needed (the empty asm keeps the
    // compiler from moving LDS accesses across the hand-over).
    auto stage = [&](int c) {
#pragma unroll
        for (int m = 0; m < 16; ++m) *reinterpret_cast<u4v *>(xs + ((m + rot) & 15) * kXRow + 8 * threadIdx.x) = xr[m];
        if (D > 0) fetch_x(c + 1);
        asm volatile("" ::: "memory");
    };
    stage(0);
    half8 A[16];
    // D = 0 has exactly one chunk: a literal trip count of one, so that nothing of the tile
    // loop (the sign expansions) is hoisted out of it and kept live for every tile at once
    const int nloop = D > 0 ? nchunk : 1;
    for (int c0 = 0; c0 < nloop; c0 += DS) {
#pragma unroll
        for (int d = 0; d < DS; ++d) {
            const int c = c0 + d;
            if (c >= nloop) break;                    // uniform
            // this wave's A operands for chunk c: 8 activations of each token row per MFMA
            const uint16_t *xa = xs + n * kXRow + 128 * (4 * wave + b);
#pragma unroll
            for (int j = 0; j < 16; ++j) A[j] = *reinterpret_cast<const half8 *>(xa + 8 * j);
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                SmSlot &sl = ring[d][t];
                const uint32_t sbits = sl.s & 0xFFFFu;
                const uint32_t s2abs = (sbits & 0x7FFFu) * 0x00010001u;
                const uint32_t flip = (sbits & 0x8000u) ? 0u : 0xFFFFFFFFu;   // bit 1: negative product
                const u4v w = sl.w;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t nw = w[j] ^ flip;
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[4 * j + 0], expand_q<0>(nw, s2abs), acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[4 * j + 1], expand_q<1>(nw, s2abs), acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[4 * j + 2], expand_q<2>(nw, s2abs), acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[4 * j + 3], expand_q<3>(nw, s2abs), acc[t], 0, 0, 0);
                }
                if (D > 0) issue(tl[t], c + D, sl);       // past the last chunk: no traffic
                __builtin_amdgcn_sched_barrier(0);        // tiles one after another: bounded registers
            }
            if (D > 0) {                              // compile-time
                asm volatile("" ::: "memory");     // this wave's A of chunk c is in registers
                stage(c + 1);
            }
        }
    }
    // merge the waves' K-slices.  D layout: lane (n, b) holds tokens 4b..4b+3 of row n.  Each
    // wave stores its tiles whole (conflict-free 16-byte stores); reader q of a tile takes
    // row (q >> 2) & 15, token 4 (q >> 6) + (q & 3), so a wave's reads hit 64 distinct banks
    // and its fp16 stores form 32-byte runs.
    __syncthreads();                                  // the staged x is dead from here
#pragma unroll
    for (int t = 0; t < TB; ++t)
        *reinterpret_cast<float4v *>(red + ((t * kWaves + wave) * 64 + lane) * 4) = acc[t];
    __syncthreads();
    const int q = threadIdx.x & 255, rr = (q >> 2) & 15, m = 4 * (q >> 6) + (q & 3);
#pragma unroll
    for (int t0 = 0; t0 < TB; t0 += 2) {
        const int t = t0 + (threadIdx.x >> 8);
        if (t >= TB) break;                           // uniform per wave
        const float *src = red + (t * kWaves * 64 + rr + 16 * (q >> 6)) * 4 + (q & 3);
        float v[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) v[w] = src[w * 256];
        const float tot = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
        const SmTile &T = (threadIdx.x >> 8) ? tl[t0 + 1 < TB ? t0 + 1 : t0] : tl[t0];
        const int row = T.row0 + rr;
        if (m < M && row < T.N) {
            if constexpr (SPLIT) part[((size_t)cw * M + m) * T.N + row] = tot;
            else T.y[(size_t)m * T.N + row] = f2h_rne(tot);
        }
    }
}

// y[i] = fp16(sum over chunks c = 0, 1, ... of part[c][i]), in that fixed order (i = m * N + n).
__global__ __launch_bounds__(256) void smallm_reduce_kernel(const float *__restrict__ part, int nchunk, int MN,
                                                            uint16_t *__restrict__ y)
{
    const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
    if (i >= MN) return;
    float acc = part[i];
    for (int c = 1; c < nchunk; ++c) acc += part[(size_t)c * MN + i];
    y[i] = f2h_rne(acc);
}

template <int TB, int D>
hipError_t launch_sm(const uint16_t *x, const MxSet &set, int M, int K, int tiles, hipStream_t st, std::string *desc)
{
    static_assert(TB * 256 * kWaves * 4 <= kXBytes, "merge table fits the staging area");
    if (desc) {                                        // describe the launch instead of making it
        char buf[96];
        snprintf(buf, sizeof buf, "gemv_smallm<%d,%d> grid=%d", TB, D, (tiles + TB - 1) / TB);
        desc->append(desc->empty() ? "" : ";").append(buf);
        return hipSuccess;
    }
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&gemv_smallm_kernel<TB, D, false>), hipFuncAttributeMaxDynamicSharedMemorySize,
        kXBytes);
    if (attr != hipSuccess) return attr;
    const int grid = (tiles + TB - 1) / TB;
    hipLaunchKernelGGL((gemv_smallm_kernel<TB, D, false>), dim3(grid), dim3(64 * kWaves), kXBytes, st, x, M, K,
                       tiles / grid, tiles % grid, grid, set, nullptr);
    return hipGetLastError();
}

// K split into its 4096-wide chunks over workgroups: G tile groups per chunk (at most TB tiles of 16
// rows each), so a workgroup stages one chunk of x instead of all of them; then the reduction.
template <int TB>
hipError_t launch_sm_split(const uint16_t *x, const MxSet &set, int M, int K, int tiles, int G, float *part,
                           hipStream_t st, std::string *desc)
{
    static_assert(TB * 256 * kWaves * 4 <= kXBytes, "merge table fits the staging area");
    const int nchunk = (K + kChunkK - 1) / kChunkK, MN = M * set.N[0];
    if (desc) {
        char buf[128];
        snprintf(buf, sizeof buf, "gemv_smallm_split<%d> grid=%d;smallm_reduce grid=%d", TB, G * nchunk,
                 (MN + 255) / 256);
        desc->append(desc->empty() ? "" : ";").append(buf);
        return hipSuccess;
    }
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&gemv_smallm_kernel<TB, 0, true>), hipFuncAttributeMaxDynamicSharedMemorySize,
        kXBytes);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((gemv_smallm_kernel<TB, 0, true>), dim3(G * nchunk), dim3(64 * kWaves), kXBytes, st, x, M, K,
                       tiles / G, tiles % G, G, set, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_smallm_reduce(part, nchunk, MN, set.y[0], st);
}

}  // namespace

hipError_t launch_smallm_reduce(const float *part, int nchunk, int MN, uint16_t *y, hipStream_t st)
{
    hipLaunchKernelGGL(smallm_reduce_kernel, dim3((MN + 255) / 256), dim3(256), 0, st, part, nchunk, MN, y);
    return hipGetLastError();
}

size_t smallm_split_bytes(int M, int K, int N)
{
    const int nchunk = (K + kChunkK - 1) / kChunkK;
    if (M < 2 || M > 16 || nchunk < 2 || N < 1) return 0;
    return ((size_t)nchunk * M * N * 4 + 255) & ~(size_t)255;
}

hipError_t launch_gemv_smallm(const uint16_t *x, const MxSet &set0, int M, int K, hipStream_t st, std::string *desc,
                              float *part)
{
    if (mxm_handles(M, K, set0, part != nullptr)) return launch_gemv_mxm(x, set0, M, K, st, desc, part);
    if (mx_tokens_handles(M, K, set0)) return launch_gemv_mx(x, set0, K, st, desc, M);
    MxSet set = set0;
    int tiles = 0;
    for (int i = 0; i < set.count; ++i) {
        tiles += (set.N[i] + 15) / 16;
        set.tile_end[i] = tiles;
    }
    const int per = (tiles + 255) / 256, nchunk = (K + kChunkK - 1) / kChunkK;
    if (part && set.count == 1 && nchunk > 1) {
        // one chunk per workgroup: as many tile groups per chunk as fill the 256 CUs once (a
        // workgroup holds a whole chunk of x in LDS, so one fits a CU), at most 8 tiles each
        int G = 256 / nchunk;
        if (G < 1) G = 1;
        if (G > tiles) G = tiles;
        int tb = (tiles + G - 1) / G;
        if (tb > 8) {
            tb = 8;
            G = (tiles + 7) / 8;
        }
        if (tb <= 1) return launch_sm_split<1>(x, set, M, K, tiles, G, part, st, desc);
        if (tb <= 2) return launch_sm_split<2>(x, set, M, K, tiles, G, part, st, desc);
        if (tb <= 4) return launch_sm_split<4>(x, set, M, K, tiles, G, part, st, desc);
        return launch_sm_split<8>(x, set, M, K, tiles, G, part, st, desc);
    }
    // TB tiles per workgroup: as few as fill the 256 CUs in one round, at most 6 (the grid
    // grows past 256 beyond that); with several K chunks, more chunks per tile are in flight
    if (nchunk == 1) {
        if (per <= 2) return launch_sm<2, 0>(x, set, M, K, tiles, st, desc);
        if (per <= 4) return launch_sm<4, 0>(x, set, M, K, tiles, st, desc);
        return launch_sm<6, 0>(x, set, M, K, tiles, st, desc);
    }
    if (per <= 1) return launch_sm<1, 4>(x, set, M, K, tiles, st, desc);
    if (per <= 2) return launch_sm<2, 3>(x, set, M, K, tiles, st, desc);
    return launch_sm<4, 2>(x, set, M, K, tiles, st, desc);
}

}  // namespace bin1
