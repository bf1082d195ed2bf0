// gemv_mxm.hip -- small-batch decode product (2 <= M <= 8 tokens) on the block-scaled matrix cores.
//
// y[m][n] = sum_k s[n][k/128] * w(n,k) * x[m][k] ["Bonsai 27B" page, section "Binary weight
// format", eq. b_eff], decoded inside the product with fp32 accumulation ["Bonsai 27B" page,
// section "Low-bit kernels for hybrid attention"]; a few tokens at once are what a speculative
// decoder's verification pass multiplies ["Bonsai 27B" page, section "DSpark"].
//
// The batch-1 kernel's arithmetic, with the tokens as MFMA rows.  One
// v_mfma_scale_f32_16x16x128_f8f6f4 covers ONE scale group (128 weights) of 16 weight rows:
//  * B: lane (n, g) supplies word g of the group for row n, expanded to 32 fp4 values +-1 (two
//    operations per 8 weights).  A lane loads 32 contiguous bytes of its row (two groups), so the
//    four lanes of a row swap words (a 4 x 4 transpose with two permlane32 and two permlane16
//    swaps per register quadruple) to put word g of every group in lane g.
//  * A: rows 4t + r hold limb r of token t's activations (three e4m3 limbs, row 4t + 3 zero),
//    stored in LDS in k order (a row is the group's 128 k, byte j of K-block b pairing with bit
//    4 (j % 8) + j / 8 of word b, the order unpack_fp4 gives the weights),
//    four tokens per instruction, with one E8M0 exponent per (token, group): x = 2^(e-7)
//    (L0 + L1/16 + L2/256), e the exponent of the group's largest magnitude.  An element within
//    2^10 of that maximum is exact, none is off by more than 2^-25 of it.
//  * C: lane (n, g) receives the three limb partials of token 4b + g for row n; the group scale is
//    applied with one fma.
// So up to four tokens cost one instruction per group and 16 rows, as many as batch 1.
//
// Work: a workgroup is 4 waves; wave w owns the 1024-wide pair w of the workgroup's 4096-wide K
// chunk (K <= 4096, or one chunk per workgroup with the split: fp32 partial sums per chunk, then
// the fixed-order chunk reduction of the fp16 small-batch kernel).  The wave converts its pair of
// every token into limbs once (through a wave-private LDS area) and keeps the A operands in
// registers; its tiles' weights stream through a ring of P slots.  The waves' partial rows are
// merged through LDS at the end, in a fixed order.
#include <cstdio>
#include <string>

#include "common.hpp"
#include "kernels.hpp"
#include "mx_common.hpp"

namespace bin1 {

namespace {

using namespace mx;

constexpr int kRowB = 144;                         // LDS bytes per A row: 4 K-blocks x 32 + 16 pad
constexpr int kABlk = 16 * kRowB;                  // one group's A operand (16 rows)
constexpr int kStage = 8 * kABlk + 8 * 16 + 32;    // per wave: 8 groups' A, their exponent bytes, zeros
constexpr int kStageSc = 8 * kABlk;                // offset of the exponent bytes [8 groups][16 rows]
constexpr int kStageZero = kStageSc + 8 * 16;      // offset of 32 zero bytes
constexpr int kChunk = 4096;                       // K per workgroup pass: 4 waves x 1024
constexpr size_t kMaxLds = 160 * 1024;

// After the swaps, register j of lane (n, g) holds word g of the group lane (n, j) loaded.
__device__ __forceinline__ u4v transpose4(u4v v)
{
    const auto xz = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
    const auto yw = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
    const auto xy = __builtin_amdgcn_permlane16_swap(xz[0], yw[0], false, false);
    const auto zw = __builtin_amdgcn_permlane16_swap(xz[1], yw[1], false, false);
    return u4v{xy[0], xy[1], zw[0], zw[1]};
}

// Limbs of 16 activations of one token into the A rows 4t' + r of a group's block: bytes of
// K-block kb, half h.  mx: the largest magnitude of the token's group.  Element i of the half sits
// at byte 8 (i % 4) + 4 h + i / 4 of the K-block, the order unpack_fp4 gives the weights.
__device__ __forceinline__ void convert_tok(const u4v p0, const u4v p1, float mx, uint8_t *blk, int tp, int kb, int h,
                                            uint8_t *scrow)
{
    const uint32_t hw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    float u[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) u[i] = h2f((uint16_t)(hw[i >> 1] >> (16 * (i & 1))));
    const int e0 = mx > 0.f ? __builtin_amdgcn_frexp_expf(mx) - 1 : 0;   // 2^e0 <= mx
    const float mul = __builtin_ldexpf(1.0f, 7 - e0);
#pragma unroll
    for (int i = 0; i < 16; ++i) u[i] *= mul;       // |u| < 256, exact
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        int d[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int v = __builtin_amdgcn_cvt_pk_fp8_f32(u[c], u[4 + c], 0, false);
            d[c] = __builtin_amdgcn_cvt_pk_fp8_f32(u[8 + c], u[12 + c], v, true);
            *reinterpret_cast<int *>(blk + (4 * tp + r) * kRowB + 32 * kb + (2 * c + h) * 4) = d[c];
        }
        if (r < 2) {
            // next limb: 16 (u - q), exact (q is u rounded to 4 significant bits)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                u[c] = fmaf(u[c], 16.f, -16.f * __builtin_amdgcn_cvt_f32_fp8(d[c], 0));
                u[4 + c] = fmaf(u[4 + c], 16.f, -16.f * __builtin_amdgcn_cvt_f32_fp8(d[c], 1));
                u[8 + c] = fmaf(u[8 + c], 16.f, -16.f * __builtin_amdgcn_cvt_f32_fp8(d[c], 2));
                u[12 + c] = fmaf(u[12 + c], 16.f, -16.f * __builtin_amdgcn_cvt_f32_fp8(d[c], 3));
            }
        }
    }
    if (scrow) {                                    // one lane per group: the rows' exponent bytes
        const uint32_t e = (uint32_t)(127 + e0 - 7);
        *reinterpret_cast<uint32_t *>(scrow + 4 * tp) = e | (e - 4) << 8 | (e - 8) << 16 | 127u << 24;
    }
}

struct MSlot {
    u4v w0, w1;     // 32 bytes of the lane's row: groups 2g and 2g + 1 of the pair
    u4v s;          // the row's 8 scales of the pair
};

struct MTile {
    const uint32_t *W;
    const uint16_t *S;
    uint16_t *y;
    int row0, N;
};

template <int MB, int P, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemv_mxm_kernel(const uint16_t *__restrict__ x, int M, int K, int tq, int tr, int G, MxSet set,
                     float *__restrict__ part)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int wpr = K >> 5, spr = K >> 7;
    // SPLIT: workgroup b takes K chunk b / G for tile group b % G
    const int cw = SPLIT ? (int)blockIdx.x / G : 0;
    const int gid = (int)blockIdx.x - cw * G;
    const int nb = tq + (gid < tr ? 1 : 0);
    const int pr = 4 * cw + wave;                    // this wave's 1024-wide pair
    const bool live = pr * 1024 < K;                 // wave-uniform

    // x: 16 activations of every token of the first token block(s), this lane's share of the pair
    const __amdgpu_buffer_rsrc_t rx = rsrc(x, (unsigned)M * (unsigned)K * 2u);
    u4v xr[MB][4][2];
    {
        const unsigned base = live ? (unsigned)(pr * 1024 + 16 * lane) * 2u : kOob;
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const unsigned o = base == kOob ? kOob : base + (unsigned)(4 * b + t) * (unsigned)K * 2u;
                xr[b][t][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, 0);
                xr[b][t][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, o == kOob ? kOob : o + 16u, 0, 0);
            }
    }
    __builtin_amdgcn_sched_barrier(0);

    // lane t resolves the workgroup's tile t (matrix, first row) with vector selects
    MTile tabl;
    {
        const int tile = gid + lane * G;
        const int m1 = set.count > 1 && tile >= set.tile_end[0], m2 = set.count > 2 && tile >= set.tile_end[1],
                  m3 = set.count > 3 && tile >= set.tile_end[2];
        auto sel = [&](auto a0, auto a1, auto a2, auto a3) { return m3 ? a3 : m2 ? a2 : m1 ? a1 : a0; };
        tabl.row0 = (tile - sel(0, set.tile_end[0], set.tile_end[1], set.tile_end[2])) * 16;
        tabl.N = lane < nb ? sel(set.N[0], set.N[1], set.N[2], set.N[3]) : 0;
        tabl.W = sel(set.W[0], set.W[1], set.W[2], set.W[3]);
        tabl.S = sel(set.S[0], set.S[1], set.S[2], set.S[3]);
        tabl.y = sel(set.y[0], set.y[1], set.y[2], set.y[3]);
    }
    auto rlp = [](const void *p, int t) {
        const unsigned long long v = reinterpret_cast<unsigned long long>(p);
        const unsigned lo = (unsigned)__builtin_amdgcn_readlane((unsigned)v, t);
        const unsigned hi = (unsigned)__builtin_amdgcn_readlane((unsigned)(v >> 32), t);
        return ((unsigned long long)hi << 32) | lo;
    };
    // Ring slot fill for the workgroup's it-th tile; slots past the last tile, rows past N and a
    // pair past K load nothing (zeros).
    auto issue = [&](int it, MSlot &sl) {
        const int L = it & 63;
        const int N = it < nb ? __builtin_amdgcn_readlane(tabl.N, L) : 0;
        const int row = __builtin_amdgcn_readlane(tabl.row0, L) + n;
        const unsigned Nr = live ? (unsigned)N : 0u;
        const __amdgpu_buffer_rsrc_t rW =
            rsrc(reinterpret_cast<const void *>(rlp(tabl.W, L)), Nr * (unsigned)wpr * 4u);
        const __amdgpu_buffer_rsrc_t rS =
            rsrc(reinterpret_cast<const void *>(rlp(tabl.S, L)), Nr * (unsigned)spr * 2u);
        const unsigned ow = (mul24((unsigned)row, (unsigned)wpr) + 32u * (unsigned)pr + 8u * (unsigned)g) * 4u;
        const unsigned os = (mul24((unsigned)row, (unsigned)spr) + 8u * (unsigned)pr) * 2u;
        sl.w0 = __builtin_amdgcn_raw_buffer_load_b128(rW, ow, 0, kNT);
        sl.w1 = __builtin_amdgcn_raw_buffer_load_b128(rW, ow + 16u, 0, kNT);
        sl.s = __builtin_amdgcn_raw_buffer_load_b128(rS, os, 0, 0);
    };
    MSlot ring[P];
#pragma unroll
    for (int p = 0; p < P; ++p) issue(p, ring[p]);

    // ---- the wave's pair of x -> limbs (wave-private LDS) -> A operands in registers
    uint8_t *st = lds + wave * kStage;
    if (lane < 2) *reinterpret_cast<u4v *>(st + kStageZero + 16 * lane) = u4v{0, 0, 0, 0};
    const int gam = lane >> 3, kb = (lane & 7) >> 1, h = lane & 1;   // conversion: lane's group, K-block, half
    const int m = lane & 15, r = m & 3;                             // A operand: lane's row
    int8v A[8][MB];
    int scA[8][MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float mx = absmax16(xr[b][t][0], xr[b][t][1]);
            mx = fmaxf(mx, __shfl_xor(mx, 1, kWave));
            mx = fmaxf(mx, __shfl_xor(mx, 2, kWave));
            mx = fmaxf(mx, __shfl_xor(mx, 4, kWave));   // the whole group (8 lanes)
            convert_tok(xr[b][t][0], xr[b][t][1], mx, st + gam * kABlk, t, kb, h,
                        (lane & 7) == 0 ? st + kStageSc + 16 * gam : nullptr);
        }
        asm volatile("" ::: "memory");               // the wave's own LDS writes, then its reads
        // the fp8 A operand of a 16x16x128 product: lane (m, g) holds k = 16g .. 16g + 15 in its
        // first four registers and k = 64 + 16g .. 64 + 16g + 15 in the other four
#pragma unroll
        for (int gg = 0; gg < 8; ++gg) {
            const uint8_t *blk = st + gg * kABlk;
            const int lo = r == 3 ? kStageZero - gg * kABlk : m * kRowB + 16 * g;
            const int hi = r == 3 ? lo + 16 : lo + 64;
            const u4v a0 = *reinterpret_cast<const u4v *>(blk + lo);
            const u4v a1 = *reinterpret_cast<const u4v *>(blk + hi);
            int8v a;
            a[0] = a0.x; a[1] = a0.y; a[2] = a0.z; a[3] = a0.w;
            a[4] = a1.x; a[5] = a1.y; a[6] = a1.z; a[7] = a1.w;
            A[gg][b] = a;
            scA[gg][b] = (int)st[kStageSc + 16 * gg + m];
        }
        asm volatile("" ::: "memory");               // reads done before the next block's writes
    }

    // ---- tiles: 8 groups x MB token blocks of products per tile; partial rows to LDS
    float *red = reinterpret_cast<float *>(lds + 4 * kStage);    // [tile][MB][wave][64 lanes]
    for (int j0 = 0; j0 < nb; j0 += P) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int it = j0 + p;
            if (it >= nb) break;                      // uniform
            const u4v wa = transpose4(ring[p].w0), wb = transpose4(ring[p].w1);
            const u4v sv = ring[p].s;
            float acc[MB];
#pragma unroll
            for (int b = 0; b < MB; ++b) acc[b] = 0.f;
#pragma unroll
            for (int gg = 0; gg < 8; ++gg) {
                const uint32_t wd = (gg & 1) ? wb[gg >> 1] : wa[gg >> 1];
                const uint32_t s2 = sv[gg >> 1];
                const float s = h2f((uint16_t)((gg & 1) ? s2 >> 16 : s2 & 0xFFFFu));
                const int8v B = unpack_fp4(wd);
#pragma unroll
                for (int b = 0; b < MB; ++b) {
                    const float4v c = mma_b<0>(A[gg][b], B, scA[gg][b], float4v{0.f, 0.f, 0.f, 0.f});
                    // B held -w: the group's partial is -(L0 + L1 + L2) terms
                    acc[b] = fmaf(-s, (c[0] + c[1]) + c[2], acc[b]);
                }
            }
            if (P > 1 || it + P < nb) issue(it + P, ring[p]);
#pragma unroll
            for (int b = 0; b < MB; ++b) red[((it * MB + b) * 4 + wave) * 64 + lane] = acc[b];
        }
    }
    __syncthreads();
    // ---- merge the 4 waves (fixed order) and store: entry e = (tile, block, lane).  The entry
    // count is a multiple of 64, so a pass covers whole waves, and the table shuffles come before
    // any lane-dependent branch: a shuffle from a lane outside a branch reads 0.
    for (int e = threadIdx.x; e < nb * MB * 64; e += 256) {
        const int it = e / (MB * 64), rem = e - it * MB * 64, b = rem >> 6, l = rem & 63;
        const int L = it & 63;
        const int row = __shfl(tabl.row0, L, kWave) + (l & 15), N = __shfl(tabl.N, L, kWave);
        const unsigned long long yp =
            ((unsigned long long)(unsigned)__shfl((unsigned)(reinterpret_cast<unsigned long long>(tabl.y) >> 32), L, kWave)
             << 32) |
            (unsigned)__shfl((unsigned)reinterpret_cast<unsigned long long>(tabl.y), L, kWave);
        const float *src = red + ((it * MB + b) * 4) * 64 + l;
        const float tot = ((src[0] + src[64]) + src[128]) + src[192];
        const int tok = 4 * b + (l >> 4);
        if (tok < M && row < N) {
            if constexpr (SPLIT) part[((size_t)cw * M + tok) * N + row] = tot;
            else reinterpret_cast<uint16_t *>(yp)[(size_t)tok * N + row] = f2h_rne(tot);
        }
    }
}

constexpr size_t lds_bytes(int MB, int tiles_per_wg) { return (size_t)4 * kStage + (size_t)tiles_per_wg * MB * 1024; }

// largest tile count per workgroup the merge table and the one-per-lane tile table hold
constexpr int max_tiles(int MB)
{
    const int t = (int)((kMaxLds - (size_t)4 * kStage) / ((size_t)MB * 1024));
    return t < 64 ? t : 64;
}

template <int MB, int P, bool SPLIT>
hipError_t launch_t(const uint16_t *x, const MxSet &set, int M, int K, int tiles, int G, int nchunk, float *part,
                    hipStream_t st, std::string *desc)
{
    const int per = (tiles + G - 1) / G;
    const size_t shm = lds_bytes(MB, per);
    if (desc) {
        char buf[128];
        if (SPLIT)
            snprintf(buf, sizeof buf, "gemv_mxm_split<%d,%d> grid=%d;smallm_reduce grid=%d", MB, P, G * nchunk,
                     (M * set.N[0] + 255) / 256);
        else
            snprintf(buf, sizeof buf, "gemv_mxm<%d,%d> grid=%d", MB, P, G);
        desc->append(desc->empty() ? "" : ";").append(buf);
        return hipSuccess;
    }
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&gemv_mxm_kernel<MB, P, SPLIT>), hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)kMaxLds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((gemv_mxm_kernel<MB, P, SPLIT>), dim3(G * (SPLIT ? nchunk : 1)), dim3(256), shm, st, x, M, K,
                       tiles / G, tiles % G, G, set, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !SPLIT) return e;
    return launch_smallm_reduce(part, nchunk, M * set.N[0], set.y[0], st);
}

template <int MB, bool SPLIT>
hipError_t launch_p(const uint16_t *x, const MxSet &set, int M, int K, int tiles, int G, int nchunk, float *part,
                    hipStream_t st, std::string *desc)
{
    const int per = (tiles + G - 1) / G;
    if (per <= 1) return launch_t<MB, 1, SPLIT>(x, set, M, K, tiles, G, nchunk, part, st, desc);
    if (per <= 2) return launch_t<MB, 2, SPLIT>(x, set, M, K, tiles, G, nchunk, part, st, desc);
    return launch_t<MB, 4, SPLIT>(x, set, M, K, tiles, G, nchunk, part, st, desc);
}

}  // namespace

// The dispatch routes 2 <= M <= 8 here (mxm_handles) for tall products only: every workgroup
// first turns its pair of every token's activations into limbs (about ten VALU operations per
// element, at one wave per SIMD), which only pays off over many tiles.  Measured on the 8B step
// at M = 8 (each launch class replayed alone): lm_head (9496 tiles, 38 per workgroup) 39.3 us
// against 51.3 us on the fp16 kernel, but q|k|v 15.0 against 4.8, o 8.3 against 4.8, gate|up
// 12.5 against 9.2, down 18.5 against 9.1.
constexpr int kMxmMinTiles = 4096;

bool mxm_shape_ok(int M, int K, int count, bool have_part)
{
    if (M < 2 || M > 8 || K <= 0 || K % 1024 != 0) return false;
    return K <= kChunk || (have_part && count == 1);
}

bool mxm_handles(int M, int K, const MxSet &set, bool have_part)
{
    int tiles = 0;
    for (int i = 0; i < set.count; ++i) tiles += (set.N[i] + 15) / 16;
    return tiles >= kMxmMinTiles && mxm_shape_ok(M, K, set.count, have_part);
}

hipError_t launch_gemv_mxm(const uint16_t *x, const MxSet &set0, int M, int K, hipStream_t st, std::string *desc,
                           float *part)
{
    MxSet set = set0;
    int tiles = 0;
    for (int i = 0; i < set.count; ++i) {
        tiles += (set.N[i] + 15) / 16;
        set.tile_end[i] = tiles;
    }
    const int nchunk = (K + kChunk - 1) / kChunk;
    const bool split = nchunk > 1;
    if (!mxm_shape_ok(M, K, set.count, part != nullptr)) return hipErrorInvalidValue;
    const int MB = M <= 4 ? 1 : 2;
    const int cap = MB == 1 ? max_tiles(1) : max_tiles(2);
    // workgroups: every tile its own up to two per CU (512); past that 256 or more, as few tiles
    // each as fit the merge table.  With the split, the chunks share those workgroups.
    const int wgs = split ? (512 / nchunk > 0 ? 512 / nchunk : 1) : 512;
    int G = tiles <= wgs ? tiles : (split ? wgs : 256);
    if ((tiles + G - 1) / G > cap) G = (tiles + cap - 1) / cap;
    if (MB == 1)
        return split ? launch_p<1, true>(x, set, M, K, tiles, G, nchunk, part, st, desc)
                     : launch_p<1, false>(x, set, M, K, tiles, G, 1, part, st, desc);
    return split ? launch_p<2, true>(x, set, M, K, tiles, G, nchunk, part, st, desc)
                 : launch_p<2, false>(x, set, M, K, tiles, G, 1, part, st, desc);
}

}  // namespace bin1
