// gemv_mx.hip -- batch-1 decode GEMV on the gfx950 block-scaled matrix cores.
//
// What is computed: y[n] = sum_k s[n][k/128] * w(n,k) * x[k], w = +-1 from one bit each,
// one fp16 scale per 128 weights ["Bonsai 27B" page, section "Binary weight format",
// eq. b_eff], decoded inside the product with fp32 accumulation ["Bonsai 27B" page,
// section "Low-bit kernels for hybrid attention"]; multiply-free +-1 weights ["PrismML
// Bonsai -- 1.15GB ..." page, section "What 1-bit is"].
//
// How (MI355X-specific design):
//  * The decode GEMV is HBM-bound, so the budget is ~0.7 VALU op per weight at 8 TB/s.
//    Plain sign expansion into fp16 pairs costs ~1 op per weight.  Instead each packed
//    word becomes 32 fp4 (e2m1) values +-1 with one shift and one and-or per 8 weights
//    (the bit goes straight into the nibble's sign position), and the block-scaled MFMA
//    v_mfma_scale_f32_16x16x128_f8f6f4 does the 4096 +-x adds per instruction.
//  * The MFMA's other operand must be fp8, so each 32-element block of x is split into
//    three e4m3 limbs x = 2^(e-7) (L0 + L1/16 + L2/256) with e the block's max exponent
//    (the fourth limb row of the A operand is zero); the limb exponents go into the MFMA's
//    per-32-element E8M0 scales.  Three limbs carry 12 significant bits, more than fp16's
//    11: an element within 2^10 of its block's maximum is exact, and none is off by more
//    than 2^-25 of that maximum.  The limbs are built once per workgroup into LDS.
//  * One 16x16x128 MFMA covers 16 rows x 128 weights: lane (n, g) supplies word t of its
//    row's group g, and the 16 A rows are (group G, limb r) with A zero outside group G,
//    so C[4G+r][n] is the unscaled limb-r partial of group G -- exactly what lane (n, G)
//    holds afterwards.  The fp16 group scale is then applied with one FMA per group.
//  * Weights are streamed with nontemporal buffer loads, several row tiles ahead per wave.
//    A lane owns two adjacent scale groups (32 contiguous bytes of its row and one dword of
//    scales), so each wave reads whole 128-byte lines; the 4 waves of a workgroup split K
//    in 1024-weight "pairs" (8 groups) and combine their partial rows in LDS.  Longer rows
//    with one tile per workgroup (4096 < K <= 16384) use one wave per pair instead (8, 12 or
//    16 waves, two to four per SIMD), so no wave converts or contracts a second pair.
//  * Segment sigma (two per pair p, h = sigma % 2) is what one chain of four MFMAs covers:
//    MFMA K-block G of segment sigma is scale group gamma = 8p + 2G + h.
#include <algorithm>
#include <cstdio>
#include <string>

#include "common.hpp"
#include "kernels.hpp"
#include "mx_common.hpp"

namespace bin1 {

namespace {

using namespace mx;

// x (fp16, K values) -> fp8 limbs in the A-operand order, plus E8M0 exponents, in LDS.
// Block beta = k/32 holds the 32 activations of packed word beta (word t = beta % 4 of group
// gamma = beta / 4); within the block, element j pairs with weight bit pi(j) = 4*(j%8) + j/8
// (the order unpack_fp4 produces).  Task tau covers activations [16 tau, 16 tau + 16); thread
// t of NT takes tasks t, t+NT, ...  The x loads are issued before the weight prefetch (loads retire
// in order, so waiting on them later does not drain the prefetch).
template <int XT>
struct XLoad {
    u4v v[XT][2];
};

__device__ __forceinline__ int nseg_of(int K) { return 2 * ((K + 1023) >> 10); }

template <int XT, int NT>
__device__ __forceinline__ void x_load(int K, const uint16_t *__restrict__ x, XLoad<XT> &xl)
{
    const int tid = threadIdx.x;
    const __amdgpu_buffer_rsrc_t rx = rsrc(x, (unsigned)K * 2u);
#pragma unroll
    for (int q = 0; q < XT; ++q) {
        const unsigned off = 32u * (unsigned)(tid + NT * q);     // past K: zeros, no traffic
        xl.v[q][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
        xl.v[q][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16u, 0, 0);
    }
}

// What limbs_build leaves unwritten: the zero bytes of every block, and, when K is not a
// multiple of 1024, the last pair's two segments in full (zero limbs, unit exponents 2^0),
// so that groups past K add nothing.  Every row of a segment inside K is written by the build.
template <int NT>
__device__ __forceinline__ void limbs_fill(int K, uint8_t *lds)
{
    const int nseg = nseg_of(K);
    const int full = ((K >> 7) & 7) ? nseg - 2 : nseg;     // segments the build covers
    uint32_t *sc = reinterpret_cast<uint32_t *>(lds + nseg * 4 * kBlk);
    const int tid = threadIdx.x;
    for (int i = tid; i < nseg * 4; i += NT) *reinterpret_cast<u4v *>(lds + i * kBlk + kZero) = u4v{0, 0, 0, 0};
    u4v *tail = reinterpret_cast<u4v *>(lds + full * 4 * kBlk);
    for (int i = tid; i < (nseg - full) * 4 * kBlk / 16; i += NT) tail[i] = u4v{0, 0, 0, 0};
    for (int i = tid; i < (nseg - full) * 16; i += NT) sc[full * 16 + i] = 0x7F7F7F7Fu;
}

template <int XT, bool T2, int NT>
__device__ __forceinline__ void limbs_build(int K, uint8_t *lds, const XLoad<XT> &xl)
{
    const int nseg = nseg_of(K);
    uint32_t *sc = reinterpret_cast<uint32_t *>(lds + nseg * 4 * kBlk);
    const int tid = threadIdx.x;
    const int ntask = K >> 4;                       // even, so a 32-block's two tasks pair up
#pragma unroll
    for (int q = 0; q < XT; ++q) {
        const int tau = tid + NT * q;
        if (NT * q >= ntask) break;                   // uniform: no task of this round
        const u4v p0 = xl.v[q][0], p1 = xl.v[q][1];
        float mx = absmax16(p0, p1);
        mx = fmaxf(mx, __shfl_xor(mx, 1, kWave));        // the other half of the 32-block
        if (tau < ntask) {
            const int beta = tau >> 1, h = tau & 1;
            const int gamma = beta >> 2, t = beta & 3;
            const int sigma = 2 * (gamma >> 3) + (gamma & 1), G = (gamma & 7) >> 1;
            convert16<T2>(p0, p1, mx, lds + (sigma * 4 + t) * kBlk, G, h,
                      reinterpret_cast<uint8_t *>(sc) + (sigma * 16 + 4 * G) * 4 + t);
        }
    }
}

// The workgroup's tile table, one tile per lane: lane i describes the workgroup's i-th tile
// (16*R rows) -- its matrix's weights, scales, output and row count, and its first row --
// computed with vector selects once per kernel.  Uniform reads (readlane with a scalar lane
// index) put a tile's entry in scalar registers; indexing the kernel argument by a computed
// matrix index instead costs a scalar-memory round trip per tile.
struct TileTab {
    unsigned long long W, S, y;
    int row0, N;
};

typedef int int4v __attribute__((ext_vector_type(4)));
constexpr int kTabBytes = 64 * 16;                   // the merge's copy of the table in LDS

template <int R>
__device__ __forceinline__ TileTab tile_tab(const MxSet &set, int tile)
{
    const int m1 = set.count > 1 && tile >= set.tile_end[0], m2 = set.count > 2 && tile >= set.tile_end[1],
              m3 = set.count > 3 && tile >= set.tile_end[2];
    auto sel = [&](auto a0, auto a1, auto a2, auto a3) { return m3 ? a3 : m2 ? a2 : m1 ? a1 : a0; };
    TileTab t;
    t.row0 = (tile - sel(0, set.tile_end[0], set.tile_end[1], set.tile_end[2])) * 16 * R;
    t.N = sel(set.N[0], set.N[1], set.N[2], set.N[3]);
    t.W = (unsigned long long)sel(set.W[0], set.W[1], set.W[2], set.W[3]);
    t.S = (unsigned long long)sel(set.S[0], set.S[1], set.S[2], set.S[3]);
    t.y = (unsigned long long)sel(set.y[0], set.y[1], set.y[2], set.y[3]);
    return t;
}

// The same for a launch of at most two matrices, from scalar kernel arguments (no argument-table
// loads); the output pointer is filled in later, for the merge.
template <int R>
__device__ __forceinline__ TileTab tile_tab2(const uint32_t *W0, const uint16_t *S0, int N0, int te0,
                                             const uint32_t *W1, const uint16_t *S1, int N1, int tile)
{
    const bool m1 = tile >= te0;
    TileTab t;
    t.row0 = (tile - (m1 ? te0 : 0)) * 16 * R;
    t.N = m1 ? N1 : N0;
    t.W = (unsigned long long)(m1 ? W1 : W0);
    t.S = (unsigned long long)(m1 ? S1 : S0);
    t.y = 0;
    return t;
}

__device__ __forceinline__ int lane_of(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

__device__ __forceinline__ unsigned long long lane_of(unsigned long long v, int l)
{
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((unsigned)v, l);      // int result:
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((unsigned)(v >> 32), l);   // no sign extension
    return ((unsigned long long)hi << 32) | lo;
}

// One ring slot: for each 16-row block r and each of the wave's pairs, 32 bytes of weights
// (groups gamma0, gamma0+1) and their two scales (one dword; or two halves when K/128 is odd,
// where a dword load could straddle rows misaligned).
template <int SP, int R, bool T2>
struct Slot {
    u4v w[R][SP][2][T2 ? 2 : 1];        // per group: 4 binary words, or 8 ternary words
    uint32_t s[R][SP];
    uint16_t s1[R][SP];
};

template <int SP, int P, int R, bool ODD, bool T2, int NW, bool TWO, int TT, bool AL>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, 4)))
void gemv_mx_kernel(const uint16_t *__restrict__ x, int Ktq, int trg, const uint32_t *W0, const uint16_t *S0,
                    const uint32_t *W1, const uint16_t *S1, int N0, int N1, MxSet set)
{
    const int K = Ktq & 0xFFFF, tq = (Ktq >> 16) & 0xFF, tr = trg & 0xFFFF, grid = trg >> 16;
    // Several tokens (2 <= M <= 8): the grid holds one copy of the one-token grid per token, and
    // workgroup b serves token b / grid with the one-token work of workgroup b % grid.
    const int mt1 = (Ktq >> 24) & 7;                  // tokens - 1
    int token = 0;
    for (int j = 1; j <= mt1; ++j) token += blockIdx.x >= (unsigned)(j * grid) ? 1 : 0;
    const unsigned bid = blockIdx.x - (unsigned)(token * grid);
    x += (size_t)token * K;
    const int te0 = (N0 + 16 * R - 1) / (16 * R);   // matrix 0's tiles
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);      // wave-uniform
    const int n = lane & 15, g = lane >> 4;
    // TT groups of NWP waves: wave group tt takes the workgroup's tiles tt, tt + TT, ..., and
    // wave wp of a group the 1024-wide pairs wp, wp + NWP, ... of each; all waves share one
    // conversion of x to limbs (so a CU converts x once for all its tiles)
    static_assert(NW % TT == 0 && (NW / TT) % 4 == 0 && (TT == 1 || TWO), "wave groups of 4k waves");
    constexpr int NWP = NW / TT;
    const int tt = wave / NWP, wp = wave - tt * NWP;                 // wave-uniform
    constexpr int NT = 64 * NW;                      // threads
    const int npair = (K + 1023) >> 10, nseg = 2 * npair;
    const int wpr = T2 ? K >> 4 : K >> 5, spr = K >> 7;   // words per row: 16 or 32 weights each
    constexpr int kGW = T2 ? 8 : 4;                      // words per scale group
    // The scalars come first in the argument list so that they arrive preloaded in registers
    // (14 dwords, what the hardware preloads: K and tq, tr and the grid size packed in halves;
    // the first two matrices' pointers and row counts): the tile count is split on the host
    // (tiles = tq * grid + tr), so no load of the grid size and no division sit in front of the
    // first loads.  With at most two matrices (TWO) the whole tile table comes from these
    // scalars; otherwise a workgroup whose first tile is in matrix 0 starts its weight loads
    // without waiting for the argument table.
    const int my_tiles = tq + (bid < (unsigned)tr ? 1 : 0);                // <= 64

    Slot<SP, R, T2> ring[P];

    // Ring slot fill for the workgroup's it-th tile.  Slots past the last tile, rows past N
    // and groups past K get out-of-range offsets: zero data and zero scales, no traffic.
    // Row offsets use mul24 (rows < 2^24), which keeps the wait counts exact.
    auto issue_t = [&](int row0, int N, unsigned long long Wp, unsigned long long Sp, Slot<SP, R, T2> &sl) {
        const __amdgpu_buffer_rsrc_t rW = rsrc(reinterpret_cast<const void *>(Wp), (unsigned)N * (unsigned)wpr * 4u);
        const __amdgpu_buffer_rsrc_t rS = rsrc(reinterpret_cast<const void *>(Sp), (unsigned)N * (unsigned)spr * 2u);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = row0 + 16 * r + n;
            const bool rok = row < N;
#pragma unroll
            for (int q = 0; q < SP; ++q) {
                const int gam = 8 * (wp + NWP * q) + 2 * g;     // this lane's first group
                const bool ok0 = rok && gam < spr, ok1 = rok && gam + 1 < spr;
                const unsigned ow = (mul24((unsigned)row, (unsigned)wpr) + (unsigned)kGW * gam) * 4u;
                const unsigned os = (mul24((unsigned)row, (unsigned)spr) + gam) * 2u;
#pragma unroll
                for (int v = 0; v < (T2 ? 2 : 1); ++v) {
                    sl.w[r][q][0][v] = __builtin_amdgcn_raw_buffer_load_b128(rW, ok0 ? ow + 16u * v : kOob, 0, kNT);
                    sl.w[r][q][1][v] =
                        __builtin_amdgcn_raw_buffer_load_b128(rW, ok1 ? ow + 4u * kGW + 16u * v : kOob, 0, kNT);
                }
                if (ODD) {
                    sl.s[r][q] = __builtin_amdgcn_raw_buffer_load_b16(rS, ok0 ? os : kOob, 0, 0);
                    sl.s1[r][q] = __builtin_amdgcn_raw_buffer_load_b16(rS, ok1 ? os + 2u : kOob, 0, 0);
                } else {
                    sl.s[r][q] = __builtin_amdgcn_raw_buffer_load_b32(rS, ok0 ? os : kOob, 0, 0);
                }
            }
        }
    };
    // the workgroup's it-th tile from the lane table (slots past the last tile load nothing)
    auto issue = [&](const TileTab &tab, int it, Slot<SP, R, T2> &sl) {
        const int L = it & 63;
        issue_t(lane_of(tab.row0, L), it < my_tiles ? lane_of(tab.N, L) : 0, lane_of(tab.W, L), lane_of(tab.S, L), sl);
    };

    // Entry: the x loads, then the first tile's weights straight from the kernel argument
    // (most launches give a workgroup one tile, whose weight latency is then the critical
    // path), and only then the LDS fill and the lane table for the other ring slots.
    constexpr int XT = SP;                           // activation tasks per thread (K <= 1024*NW*SP)
    XLoad<XT> xl;
    x_load<XT, NT>(K, x, xl);
    __builtin_amdgcn_sched_barrier(0);               // x loads go out before the argument-table loads
    TileTab tab;
    if constexpr (TWO) {
        tab = tile_tab2<R>(W0, S0, N0, te0, W1, S1, N1, bid + lane * grid);
#pragma unroll
        for (int p = 0; p < P; ++p) issue(tab, tt + TT * p, ring[p]);
        limbs_fill<NT>(K, lds);
    } else {
        // only the scalars are chosen under the (uniform) branch: one issue after it, so no
        // load sits on either side of a join
        unsigned long long Wp = (unsigned long long)W0, Sp = (unsigned long long)S0;
        int row0 = (int)bid * 16 * R, Nt = N0;
        if (bid >= (unsigned)te0) {
            const TileTab t0 = tile_tab<R>(set, bid);
            Wp = t0.W;
            Sp = t0.S;
            row0 = t0.row0;
            Nt = t0.N;
        }
        issue_t(row0, my_tiles > 0 ? Nt : 0, Wp, Sp, ring[0]);
        limbs_fill<NT>(K, lds);
        tab = tile_tab<R>(set, bid + lane * grid);
#pragma unroll
        for (int p = 1; p < P; ++p) issue(tab, p, ring[p]);
    }
    // The fill and the build write disjoint bytes unless the last pair is partial (the fill then
    // zeroes the build's last segments first): only then must the fill be complete before it.
    if ((K >> 7) & 7) __syncthreads();
    limbs_build<XT, T2, NT>(K, lds, xl);
    __syncthreads();                                  // limbs visible

    const uint32_t *sc = reinterpret_cast<const uint32_t *>(lds + nseg * 4 * kBlk);
    // after the limbs: the tile table for the merge (64 entries of row0, N, output pointer), then
    // the merge table
    int4v *tabl = reinterpret_cast<int4v *>(lds + nseg * (4 * kBlk + 64));
    float *red = reinterpret_cast<float *>(lds + nseg * (4 * kBlk + 64) + kTabBytes);
    const int m = lane & 15, G = m >> 2;
    const int lo = (G == (g >> 1)) ? m * 32 + 16 * (g & 1) : kZero;
    const int hi = (G == 2 + (g >> 1)) ? m * 32 + 16 * (g & 1) : kZero;

    // The wave's A operands (its K-slice of the limbs) stay in registers for the whole
    // kernel: 8 x 8 registers per pair, read from LDS once.  AL: only one pair's operands are
    // held, read from LDS where the pair's products run (long rows with one tile per workgroup:
    // the registers of the other pairs let more waves share a CU).
    int8v A[AL ? 1 : SP][2][4];
    int scA[AL ? 1 : SP][2];
    if constexpr (!AL)
#pragma unroll
    for (int q = 0; q < SP; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int sigma = 2 * (wp + NWP * q) + h;
            const bool v = wp + NWP * q < npair;
            const uint8_t *blk = lds + (v ? sigma : 0) * 4 * kBlk;
#pragma unroll
            for (int t = 0; t < 4; ++t) A[q][h][t] = load_a(blk + t * kBlk, lo, hi);
            scA[q][h] = (int)sc[(v ? sigma : 0) * 16 + m];
        }

    // Main loop: no cross-wave synchronisation.  Each wave streams its K-slice of every tile
    // of its group and parks its partial row sums in LDS; one barrier at the end merges the
    // slices and writes y with coalesced stores.  Local tile j of the group is the workgroup's
    // tile tt + TT j.
    for (int j0 = 0; tt + TT * j0 < my_tiles; j0 += P) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int it = tt + TT * (j0 + p);
            if (it >= my_tiles) goto done;            // uniform; the slots left hold dead loads
            float acc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
            for (int q = 0; q < SP; ++q) {
                const int pr = wp + NWP * q;
                if (pr < npair) {                     // wave-uniform
                    const int gam = 8 * pr + 2 * g;
                    if constexpr (AL) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const uint8_t *blk = lds + (2 * pr + h) * 4 * kBlk;
#pragma unroll
                            for (int t = 0; t < 4; ++t) A[0][h][t] = load_a(blk + t * kBlk, lo, hi);
                            scA[0][h] = (int)sc[(2 * pr + h) * 16 + m];
                        }
                    }
                    const int qa = AL ? 0 : q;        // the pair's operands
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const uint32_t sv = ring[p].s[r][q];
                        const float s0 = h2f((uint16_t)(sv & 0xFFFFu));
                        const float s1 = ODD ? h2f(ring[p].s1[r][q])
                                             : (gam + 1 < spr ? h2f((uint16_t)(sv >> 16)) : 0.f);
                        // the two segments' chains of four products each, interleaved (independent
                        // accumulators keep the matrix pipe busy); group partials added in segment order
                        float4v ca = {0.f, 0.f, 0.f, 0.f}, cb = {0.f, 0.f, 0.f, 0.f};
                        if constexpr (T2) {
                            // MFMA t takes the group's words 2t and 2t + 1 (32 weights)
                            const u4v a0 = ring[p].w[r][q][0][0], a1 = ring[p].w[r][q][0][T2 ? 1 : 0];
                            const u4v b0 = ring[p].w[r][q][1][0], b1 = ring[p].w[r][q][1][T2 ? 1 : 0];
                            ca = mma_b<0>(A[qa][0][0], unpack_t2(a0.x, a0.y), scA[qa][0], ca);
                            cb = mma_b<0>(A[qa][1][0], unpack_t2(b0.x, b0.y), scA[qa][1], cb);
                            ca = mma_b<1>(A[qa][0][1], unpack_t2(a0.z, a0.w), scA[qa][0], ca);
                            cb = mma_b<1>(A[qa][1][1], unpack_t2(b0.z, b0.w), scA[qa][1], cb);
                            ca = mma_b<2>(A[qa][0][2], unpack_t2(a1.x, a1.y), scA[qa][0], ca);
                            cb = mma_b<2>(A[qa][1][2], unpack_t2(b1.x, b1.y), scA[qa][1], cb);
                            ca = mma_b<3>(A[qa][0][3], unpack_t2(a1.z, a1.w), scA[qa][0], ca);
                            cb = mma_b<3>(A[qa][1][3], unpack_t2(b1.z, b1.w), scA[qa][1], cb);
                            acc[r] = fmaf(s0, (ca[0] + ca[1]) + (ca[2] + ca[3]), acc[r]);
                            acc[r] = fmaf(s1, (cb[0] + cb[1]) + (cb[2] + cb[3]), acc[r]);
                        } else {
                            const u4v wa = ring[p].w[r][q][0][0], wb = ring[p].w[r][q][1][0];
                            ca = mma<0>(A[qa][0][0], wa.x, scA[qa][0], ca);
                            cb = mma<0>(A[qa][1][0], wb.x, scA[qa][1], cb);
                            ca = mma<1>(A[qa][0][1], wa.y, scA[qa][0], ca);
                            cb = mma<1>(A[qa][1][1], wb.y, scA[qa][1], cb);
                            ca = mma<2>(A[qa][0][2], wa.z, scA[qa][0], ca);
                            cb = mma<2>(A[qa][1][2], wb.z, scA[qa][1], cb);
                            ca = mma<3>(A[qa][0][3], wa.w, scA[qa][0], ca);
                            cb = mma<3>(A[qa][1][3], wb.w, scA[qa][1], cb);
                            // B held -w, so a group's partial is -(c0+c1+c2+c3)
                            acc[r] = fmaf(-s0, (ca[0] + ca[1]) + (ca[2] + ca[3]), acc[r]);
                            acc[r] = fmaf(-s1, (cb[0] + cb[1]) + (cb[2] + cb[3]), acc[r]);
                        }
                    }
                }
            }
            // refill the slot with the group's tile P further on; with a one-slot ring only when
            // there is one (the branch is uniform, and nothing after it waits on other loads)
            const int nxt = tt + TT * (j0 + p + P);
            if (P > 1 || nxt < my_tiles) issue(tab, nxt, ring[p]);
            float *rb = red + it * (16 * NWP * R);    // [tile][16R rows][NWP waves]
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float v = sum_groups(acc[r]);
                if (lane < 16) rb[(16 * r + lane) * NWP + wp] = v;
            }
        }
    }
done:
    if constexpr (TWO) {                              // the outputs, for the merge
        const int tile = bid + lane * grid;
        tab.y = (unsigned long long)(tile >= te0 ? set.y[1] : set.y[0]);
    }
    if (wave == 0) tabl[lane] = int4v{tab.row0, tab.N, (int)(unsigned)tab.y, (int)(unsigned)(tab.y >> 32)};
    __syncthreads();
    // Merge: thread t finishes rows t, t+NT, ... of the workgroup's tiles in order, with the
    // tile's entry read from the LDS table (per lane: no lane depends on another being active).
    // The empty asm takes the entry and the partials together, so both LDS reads are issued
    // before one wait (left alone, the compiler moves the partials' read into the store's
    // branch, behind the entry's wait).
    for (int e = tid; e < my_tiles * 16 * R; e += NT) {
        const int it = e / (16 * R), j = e - it * (16 * R);
        const int4v t = tabl[it];
        float4v pr[NWP / 4];                          // waves 4.. of a wider pair split in pr[1]
#pragma unroll
        for (int v = 0; v < NWP / 4; ++v) pr[v] = *reinterpret_cast<const float4v *>(red + e * NWP + 4 * v);
#pragma unroll
        for (int v = 0; v < NWP / 4; ++v) asm volatile("" ::"v"(pr[v]));
        asm volatile("" ::"v"(t));
        float tot = (pr[0][0] + pr[0][1]) + (pr[0][2] + pr[0][3]);
#pragma unroll
        for (int v = 1; v < NWP / 4; ++v) tot += (pr[v][0] + pr[v][1]) + (pr[v][2] + pr[v][3]);
        const int row = t[0] + j;
        if (row < t[1])
            reinterpret_cast<uint16_t *>(((unsigned long long)(unsigned)t[3] << 32) | (unsigned)t[2])
                [(size_t)token * t[1] + row] = f2h_rne(tot);                 // y: [tokens][N]
    }
}

constexpr int kMaxPairs = 20;                         // K <= 20480 (A operands fit in registers)
constexpr int kMaxTileRows = 2048;                     // rows per workgroup held in the merge table
constexpr size_t kMaxLds = 160 * 1024;                 // LDS per workgroup on gfx950
// LDS: limb blocks and exponents for K, the tile table, then the merge table
// [tile][16R rows][NW waves] fp32.
constexpr size_t shm_bytes(int K, int rows_per_wg, int NW)
{
    return (size_t)(2 * ((K + 1023) >> 10)) * (4 * kBlk + 64) + kTabBytes + (size_t)rows_per_wg * NW * 4;
}

template <int SP, int P, int R, bool ODD, bool T2, int NW, bool TWO, int TT, bool AL>
hipError_t launch_mx_t(const uint16_t *x, const MxSet &set0, int K, int mt, hipStream_t st, std::string *desc)
{
    constexpr int NWP = NW / TT;
    MxSet set = set0;
    int tiles = 0;
    for (int i = 0; i < set.count; ++i) {
        tiles += (set.N[i] + 16 * R - 1) / (16 * R);
        set.tile_end[i] = tiles;
    }
    // Resident workgroups per CU follow the register budget (A operands dominate it: three
    // fit at one pair per wave, two at two); a workgroup of several wave groups fills a CU by
    // itself.  The grid grows past that only when a workgroup's rows would overflow the merge
    // table.
    const int cap = TT > 1 ? 256
                  : NW == 4 ? (SP == 1 ? 3 * 256 : SP == 2 ? 2 * 256 : 256) : (NW == 8 && SP == 1 ? 2 * 256 : 256);
    // tiles per workgroup: at most what the one-per-lane tile table holds, and what the merge
    // table holds (kMaxTileRows, and the LDS left after this K's limbs)
    constexpr int kMaxT = kMaxTileRows / (16 * R) < 64 ? kMaxTileRows / (16 * R) : 64;
    const int ldsT = (int)((kMaxLds - shm_bytes(K, 0, NWP)) / ((size_t)16 * R * NWP * 4));
    const int maxT = ldsT < kMaxT ? ldsT : kMaxT;
    const int need = (tiles + maxT - 1) / maxT, units = (tiles + TT - 1) / TT;
    const int grid = units < cap ? units : (need > cap ? need : cap);
    const int rows_per_wg = (tiles + grid - 1) / grid * 16 * R;
    const size_t shm = shm_bytes(K, rows_per_wg, NWP);
    if (shm > kMaxLds) return hipErrorInvalidValue;
    const bool two = set.count == 2;
    if (desc) {                                        // describe the launch instead of making it
        char buf[160];
        char tok[16] = "";
        if (mt > 1) snprintf(tok, sizeof tok, " tokens=%d", mt);
        if (TT > 1 || AL)
            snprintf(buf, sizeof buf, "gemv_mx<%d,%d,%d,%d,%d,%d,%d,%d%s>%s lds=%zu grid=%d", SP, P, R, (int)ODD,
                     (int)T2, NW, (int)TWO, TT, AL ? ",AL" : "", tok, shm, grid * mt);
        else
            snprintf(buf, sizeof buf, "gemv_mx<%d,%d,%d,%d,%d,%d,%d>%s lds=%zu grid=%d", SP, P, R, (int)ODD, (int)T2,
                     NW, (int)TWO, tok, shm, grid * mt);
        desc->append(desc->empty() ? "" : ";").append(buf);
        return hipSuccess;
    }
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&gemv_mx_kernel<SP, P, R, ODD, T2, NW, TWO, TT, AL>),
        hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)std::min<size_t>(shm_bytes(kMaxPairs * 1024, kMaxTileRows, NWP), kMaxLds));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((gemv_mx_kernel<SP, P, R, ODD, T2, NW, TWO, TT, AL>), dim3(grid * mt), dim3(64 * NW),
                       shm, st, x, K | (tiles / grid) << 16 | (mt - 1) << 24, (tiles % grid) | grid << 16,
                       set.W[0], set.S[0], two ? set.W[1] : nullptr, two ? set.S[1] : nullptr, set.N[0],
                       two ? set.N[1] : 0, set);
    return hipGetLastError();
}

// Launches of at most two matrices take their whole tile table from scalar arguments; several
// wave groups per workgroup (TT > 1) need that table, so three or four matrices fall back to one
// group of NW / TT waves.
template <int SP, int P, int R, bool ODD, bool T2, int NW = 4, int TT = 1, bool AL = false>
hipError_t launch_mx(const uint16_t *x, const MxSet &set, int K, int mt, hipStream_t st, std::string *desc)
{
    if (set.count <= 2) return launch_mx_t<SP, P, R, ODD, T2, NW, true, TT, AL>(x, set, K, mt, st, desc);
    return launch_mx_t<SP, P, R, ODD, T2, NW / TT, false, 1, AL>(x, set, K, mt, st, desc);
}

template <bool ODD, bool T2>
hipError_t dispatch_mx(const uint16_t *x, const MxSet &set, int K, int mt, hipStream_t st, std::string *desc)
{
    const int SP = (((K + 1023) >> 10) + 3) / 4;        // pairs per wave
    // One tile per workgroup (the grid covers all tiles): a one-slot ring, so that no dead
    // slots are filled on the way to the first tile.  Such launches are latency-bound (one
    // wave per SIMD), so 16-row tiles are used where they still fit one per workgroup: half
    // the work per workgroup, and co-resident workgroups hide each other's latency.
    int t16 = 0, t32 = 0;
    for (int i = 0; i < set.count; ++i) {
        t16 += (set.N[i] + 15) / 16;
        t32 += (set.N[i] + 31) / 32;
    }
    // Up to three 16-row tiles per workgroup still beat 32-row tiles (even shares, shorter
    // dependent chains); past that the larger tile wins.
    const int cap = SP == 1 ? 3 * 256 : SP == 2 ? 2 * 256 : 256;
    const bool one16 = t16 <= cap, one = t32 <= cap, few16 = t16 <= 3 * cap;
    switch (SP) {
    // Past one tile per workgroup, one workgroup per CU of three groups of four waves: x is
    // loaded and converted once per CU instead of once per co-resident workgroup.
    // Binary rows: past 256 16-row tiles, one 32-row tile per workgroup while that fits 256
    // workgroups, then three wave groups per workgroup on 16-row tiles (measured on the 8B q|k|v
    // and gate|up shapes).
    case 1:
        if (t16 > 256 && t32 <= 256) return launch_mx<1, 1, 2, ODD, T2>(x, set, K, mt, st, desc);
        if (t16 > 256 && t32 <= cap) return launch_mx<1, 1, 1, ODD, T2, 12, 3>(x, set, K, mt, st, desc);
        // Past three 16-row tiles per workgroup slot: binary rows on 32-row tiles in three wave
        // groups; ternary rows (twice the bytes) on 16-row tiles in two groups (4096 x 151936:
        // 44.1 us against 47.8 us on the binary layout, 49.3 us with a two-slot ring).
        if (!few16) {
            if constexpr (T2) return launch_mx<1, 1, 1, ODD, T2, 8, 2>(x, set, K, mt, st, desc);
            else return launch_mx<1, 1, 2, ODD, T2, 12, 3>(x, set, K, mt, st, desc);
        }
        return one16 ? launch_mx<1, 1, 1, ODD, T2>(x, set, K, mt, st, desc)
                 : one   ? launch_mx<1, 1, 2, ODD, T2, 12, 3>(x, set, K, mt, st, desc)
                         : launch_mx<1, 3, 1, ODD, T2>(x, set, K, mt, st, desc);
    // Binary weights, 5..8 pairs (K = 5120 at the 27B shapes): eight waves with one pair each on
    // 32-row tiles, up to 512 workgroups (measured: fewer, taller tiles beat 16-row ones, and beat
    // four waves with a second pair on some of them).  Ternary rows keep the layouts below.
    // One 16-row tile per workgroup: as many waves as pairs (up to 16), one pair each, so no wave
    // carries a second pair on the critical path (the wider workgroups fit fewer per CU).
    case 2:
        if constexpr (!T2)
            return t32 <= 3 * 512 ? launch_mx<1, 1, 2, ODD, T2, 8>(x, set, K, mt, st, desc)
                                  : launch_mx<1, 2, 2, ODD, T2, 8>(x, set, K, mt, st, desc);
        return one16 ? launch_mx<1, 1, 1, ODD, T2, 8>(x, set, K, mt, st, desc)
                 : one   ? launch_mx<2, 1, 2, ODD, T2>(x, set, K, mt, st, desc)
                 : few16 ? launch_mx<2, 2, 1, ODD, T2>(x, set, K, mt, st, desc) : launch_mx<2, 2, 2, ODD, T2>(x, set, K, mt, st, desc);
    case 3: return one16 ? launch_mx<1, 1, 1, ODD, T2, 12>(x, set, K, mt, st, desc)
                 : one   ? launch_mx<3, 1, 2, ODD, T2>(x, set, K, mt, st, desc) : launch_mx<3, 2, 2, ODD, T2>(x, set, K, mt, st, desc);
    // (ternary rows are twice as many bytes: 16-row tiles keep the ring in registers)
    case 4:
        if (one16) return launch_mx<1, 1, 1, ODD, T2, 16>(x, set, K, mt, st, desc);
        if constexpr (T2) return launch_mx<4, 1, 1, ODD, T2>(x, set, K, mt, st, desc);
        else return launch_mx<4, 1, 2, ODD, T2>(x, set, K, mt, st, desc);
    // 17..20 pairs (K = 17408 at the 27B shapes), binary: twelve waves of at most two pairs, each
    // pair's A operands read where they are used (AL), so the twelve waves fit a CU; 16-row tiles
    // on up to 256 workgroups with a one-slot ring while there are at most 256 32-row tiles, a
    // two-slot ring past that.  (27B down, 320 16-row tiles, replayed alone: 7.69 us per launch
    // against 8.33 on 160 workgroups of one 32-row tile and 8.56 with the two-slot ring.)
    default:
        if constexpr (T2) return launch_mx<5, 1, 1, ODD, T2>(x, set, K, mt, st, desc);
        else return t32 <= 256 ? launch_mx<2, 1, 1, ODD, T2, 12, 1, true>(x, set, K, mt, st, desc)
                               : launch_mx<2, 2, 1, ODD, T2, 12, 1, true>(x, set, K, mt, st, desc);
    }
}

}  // namespace

int mx_max_k() { return kMaxPairs * 1024; }

// Two tokens on short products: two copies of the one-token grid beat the small-batch kernels
// where the one-token grid is small (8B step, each class's launches replayed alone: o 3.70
// against 4.66 us, down (K = 12288) 7.15 against 8.75 us; q|k|v, 384 tiles, 4.77 against 4.73;
// gate|up 8.85 against 8.53).  From three tokens on, the copies cost about one one-token launch
// each and lose everywhere.
bool mx_tokens_handles(int M, int K, const MxSet &set)
{
    if (M != 2 || K > mx_max_k()) return false;
    int tiles = 0;
    for (int i = 0; i < set.count; ++i) tiles += (set.N[i] + 15) / 16;
    return tiles <= 256;
}

hipError_t launch_gemv_mx(const uint16_t *x, const MxSet &set, int K, hipStream_t st, std::string *desc, int mt)
{
    return ((K >> 7) & 1) ? dispatch_mx<true, false>(x, set, K, mt, st, desc)
                          : dispatch_mx<false, false>(x, set, K, mt, st, desc);
}

hipError_t launch_gemv_mx_t2(const uint16_t *x, const MxSet &set, int K, hipStream_t st, std::string *desc, int mt)
{
    return ((K >> 7) & 1) ? dispatch_mx<true, true>(x, set, K, mt, st, desc)
                          : dispatch_mx<false, true>(x, set, K, mt, st, desc);
}

}  // namespace bin1
