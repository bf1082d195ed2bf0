// prefill.hip -- prefill product y = x * W^T on the matrix cores.
//
// Prompt processing is compute-bound rather than bandwidth-bound ["Bonsai 27B" page,
// section "Low-bit kernels for hybrid attention"], so this is the one dense contraction:
// sign bits become fp16 +-scale operands (w = s_g * b, "Binary weight format" section,
// eq. b_eff) and are multiplied on the MFMA units with fp32 accumulation.  fp16 operands
// hold x and +-s exactly; bf16 would round both and runs at the same dense rate on gfx950.
//
// Tiling for gfx950: a 256 x 192 output tile per workgroup (M=2048, N=12288 gives 512
// workgroups, two full rounds over 256 CUs); four waves of 128 x 96, each a 4 x 3 grid of
// v_mfma_f32_32x32x16_f16 accumulators (192 AGPRs).  K advances 128 (one scale group) per step,
// in eight 16-wide substeps.
//
//  * Activations go through LDS (two buffers, one barrier per step): the next step's 16-byte
//    chunks are prefetched into registers and stored while the MFMAs read the current buffer.
//  * Weights never touch LDS: every wave expands the bits of its own 96 columns straight into
//    B-operand registers, one 16-wide substep ahead of the MFMAs that use them, so a
//    substep's MFMAs wait on nothing computed in it.  Within each 32-wide word the k order is permuted -- fp16 pair p of
//    a lane's operand holds bits b and b + 16 -- so one shift and one bit-field insert make
//    two +-|s| values (a negative scale is folded into the sign bits first).  The activation
//    rows are stored in LDS under the same permutation (a byte permute per dword while
//    staging), so the sum over k is unchanged.
//  * Workgroup b takes M-tile b % tiles_m: with 8 M-tiles each XCD keeps one activation
//    panel in its L2.
#include "common.hpp"
#include "kernels.hpp"

#include <cstdio>
#include <string>
#include <type_traits>

namespace bin1 {

namespace {

typedef unsigned u4v __attribute__((ext_vector_type(4)));
typedef unsigned u2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int BN = 192, BK = 128;
constexpr int LDK = BK + 8;                       // LDS row stride in halves (272 B: conflict-free)
constexpr int kRsrcFlags = 0x00020000;
constexpr unsigned kOob = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcFlags);
}

// Interleave the fp16 values of lo (k = 0..7 of a 16-wide half-word) and hi (k = 16..23 of the
// word) into the permuted order: out dword p = (lo[p], hi[p]).
__device__ __forceinline__ void interleave(const u4v lo, const u4v hi, u4v &o0, u4v &o1)
{
    o0 = u4v{__builtin_amdgcn_perm(hi.x, lo.x, 0x05040100u), __builtin_amdgcn_perm(hi.x, lo.x, 0x07060302u),
             __builtin_amdgcn_perm(hi.y, lo.y, 0x05040100u), __builtin_amdgcn_perm(hi.y, lo.y, 0x07060302u)};
    o1 = u4v{__builtin_amdgcn_perm(hi.z, lo.z, 0x05040100u), __builtin_amdgcn_perm(hi.z, lo.z, 0x07060302u),
             __builtin_amdgcn_perm(hi.w, lo.w, 0x05040100u), __builtin_amdgcn_perm(hi.w, lo.w, 0x07060302u)};
}

// Four B-operand dwords: pair p = (+-|s| for bit b0 + p, +-|s| for bit b0 + p + 16) of nw, where
// bit 1 of nw means a negative product.  bfi keeps bits 15 and 31 from the shifted word.
template <int B0>
__device__ __forceinline__ half8v expand_pairs(uint32_t nw, uint32_t s2abs)
{
    u4v d;
    d.x = (((nw << (15 - B0)) & 0x80008000u)) | s2abs;
    d.y = (((nw << (14 - B0)) & 0x80008000u)) | s2abs;
    d.z = (((nw << (13 - B0)) & 0x80008000u)) | s2abs;
    d.w = (((nw << (12 - B0)) & 0x80008000u)) | s2abs;
    return __builtin_bit_cast(half8v, d);
}

// Ternary (2-bit slots: low bit nonzero, high bit negative) B dwords of a 16-weight word:
// pair d = (slot d, slot d + 8) of nw.  The sign bits 2d + 1 and 2d + 17 land on bits 15 and 31
// with one shift; the nonzero bits 2d and 2d + 16, moved to bits 0 and 16, times |s| put |s|
// (or 0) into each half with one 24-bit multiply.
template <int D>
__device__ __forceinline__ uint32_t expand_t2_pair(uint32_t nw, uint32_t sabs)
{
    return ((nw << (14 - 2 * D)) & 0x80008000u) | mul24((nw >> (2 * D)) & 0x00010001u, sabs);
}

__device__ __forceinline__ half8v expand_t2(uint32_t nw, uint32_t sabs)
{
    const u4v d{expand_t2_pair<0>(nw, sabs), expand_t2_pair<1>(nw, sabs), expand_t2_pair<2>(nw, sabs),
                expand_t2_pair<3>(nw, sabs)};
    return __builtin_bit_cast(half8v, d);
}

}  // namespace

// BM x BN tile, WM x WN waves; a wave computes (BM / WM) x (BN / WN) as FI x FJ 32x32 fragments.
// WPE waves per SIMD (from one or several workgroups per CU).
// T2: ternary weights in 2-bit slots (16 per word) instead of sign bits (32 per word).
template <int BM, int WM, int WN, int WPE, bool T2>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void prefill_kernel(const uint16_t *__restrict__ x, const uint32_t *__restrict__ W,
                    const uint16_t *__restrict__ S, uint16_t *__restrict__ y, int M, int K, int N,
                    int tiles_m)
{
    constexpr int kThreads = 64 * WM * WN;
    constexpr int kAUnits = BM * 8 / kThreads;    // (row, word, half-word) staging units per thread
    constexpr int TM = BM / WM, TN = BN / WN, FI = TM / 32, FJ = TN / 32;
    constexpr int BUF_HALVES = BM * LDK;          // one activation buffer
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int bm = blockIdx.x % tiles_m, bn = blockIdx.x / tiles_m;
    const int m0 = bm * BM, n0 = bn * BN;
    const int wpr = T2 ? K >> 4 : K >> 5, spr = K >> 7, nk = K / BK;
    constexpr int kWS = T2 ? 8 : 4;                   // words of a row per K step
    const int fr = lane & 31, fh = lane >> 5;         // MFMA operand row / column and k-half

    const __amdgpu_buffer_rsrc_t rx = rsrc(x, (unsigned)M * (unsigned)K * 2u);
    const __amdgpu_buffer_rsrc_t rW = rsrc(W, (unsigned)N * (unsigned)wpr * 4u);
    const __amdgpu_buffer_rsrc_t rS = rsrc(S, (unsigned)N * (unsigned)spr * 2u);

    // ---- activation staging.  Unit i of a thread (u = t + kThreads i) is 16 permuted positions
    // (32 bytes) of a row in a step, unit index idx: binary, (word idx / 2, half idx % 2) -- the
    // 8-wide chunks h and h + 2 of that 32-weight word, interleaved; ternary, 16-weight word idx
    // -- its chunks 0 and 1, interleaved.  Eight consecutive lanes take units 0..3 of two adjacent
    // rows, so the rows' 68-dword LDS stride puts their 16-byte writes in distinct banks, and
    // four lanes read 64 contiguous bytes of a row.
    unsigned a_gofs[kAUnits];                         // byte offset of the unit in x at step 0
    int a_lofs[kAUnits];                              // half offset of the unit in an LDS buffer
#pragma unroll
    for (int i = 0; i < kAUnits; ++i) {
        const int u = t + kThreads * i, c = u >> 3;
        const int row = 2 * (c % (BM / 2)) + ((u >> 2) & 1);
        const int idx = (u & 3) + 4 * (c / (BM / 2)), wd = idx >> 1, h = idx & 1;
        const int m = m0 + row;
        const int k0 = T2 ? 16 * idx : 32 * wd + 8 * h;
        a_gofs[i] = m < M ? ((unsigned)m * (unsigned)K + (unsigned)k0) * 2u : kOob;
        a_lofs[i] = row * LDK + 16 * idx;
    }
    auto load_a1 = [&](int ks, int i, u4v (&r)[2]) {
        const bool ok = a_gofs[i] != kOob && ks < nk;
        const unsigned off = a_gofs[i] + (unsigned)(ks * BK * 2);
        r[0] = __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? off : kOob, 0, 0);
        r[1] = __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? off + (T2 ? 16u : 32u) : kOob, 0, 0);
    };
    auto store_a1 = [&](uint16_t *buf, int i, const u4v (&r)[2]) {
        u4v o0, o1;
        interleave(r[0], r[1], o0, o1);
        u4v *dst = reinterpret_cast<u4v *>(buf + a_lofs[i]);
        dst[0] = o0;
        dst[1] = o1;
    };
    auto load_a = [&](int ks, u4v (&ra)[kAUnits][2]) {
#pragma unroll
        for (int i = 0; i < kAUnits; ++i) load_a1(ks, i, ra[i]);
    };
    auto store_a = [&](uint16_t *buf, const u4v (&ra)[kAUnits][2]) {
#pragma unroll
        for (int i = 0; i < kAUnits; ++i) store_a1(buf, i, ra[i]);
    };
    // ---- weight bits of this wave's FJ column fragments: row n0 + TN wn + 32 j + fr, the four
    // (ternary: eight) words of a step and the group scale
    unsigned b_wofs[FJ], b_sofs[FJ];                   // byte offsets of this lane's rows at step 0
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
        const int n = n0 + wn * TN + 32 * j + fr;
        b_wofs[j] = n < N ? (unsigned)n * (unsigned)wpr * 4u : kOob;
        b_sofs[j] = n < N ? (unsigned)n * (unsigned)spr * 2u : kOob;
    }
    auto load_b = [&](int ks, u4v (&rw)[FJ][kWS / 4], uint32_t (&rs)[FJ]) {
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            const bool ok = b_wofs[j] != kOob && ks < nk;
#pragma unroll
            for (int v = 0; v < kWS / 4; ++v)
                rw[j][v] = __builtin_amdgcn_raw_buffer_load_b128(
                    rW, ok ? b_wofs[j] + (unsigned)(4 * kWS * ks + 16 * v) : kOob, 0, 0);
            rs[j] = __builtin_amdgcn_raw_buffer_load_b16(rS, ok ? b_sofs[j] + (unsigned)(2 * ks) : kOob, 0, 0);
        }
    };

    f16v acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // Activations are loaded one K-step (96 MFMAs per wave) before they are stored to LDS,
    // weights one step before use: every workgroup of an XCD reads the same activation panel
    // at about the same time, so a step's first touch comes from HBM.  Loads and stores are
    // unconditional (out-of-range offsets past the last step) so the loop is straight-line and
    // each wait covers only the loads it needs.
    u4v ra[kAUnits][2];
    u4v rw[FJ][kWS / 4];
    uint32_t rs[FJ];
    load_a(0, ra);
    load_b(0, rw, rs);
    store_a(lds, ra);
    __syncthreads();
    load_a(1, ra);

    // one K-step on buffer P: its weights are folded and step ks + 1's requested in their place;
    // the activations of step ks + 1 go to the other buffer and step ks + 2's are requested
    auto step = [&](int ks, auto P_c) {
        constexpr int P = decltype(P_c)::value;
        const uint16_t *cur = lds + P * BUF_HALVES;
        uint16_t *nxt = lds + (P ^ 1) * BUF_HALVES;
        // this step's weights: fold each scale's sign into the bits, shift by this lane's k-half
        uint32_t nw[FJ][kWS], s2[FJ];
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            const uint32_t sv = rs[j] & 0xFFFFu;
            if constexpr (T2) {
                // a negative scale flips every slot's negative bit; lane half fh takes slots
                // 4 fh .. 4 fh + 3 (and + 8) of each word
                const uint32_t flip = (sv & 0x8000u) ? 0xAAAAAAAAu : 0u;
                s2[j] = sv & 0x7FFFu;
#pragma unroll
                for (int v = 0; v < 8; ++v) nw[j][v] = (rw[j][v / 4][v % 4] ^ flip) >> (8 * fh);
            } else {
                const uint32_t flip = (sv & 0x8000u) ? 0u : 0xFFFFFFFFu;   // bit 1 of nw: negative product
                s2[j] = (sv & 0x7FFFu) * 0x00010001u;
#pragma unroll
                for (int v = 0; v < 4; ++v) nw[j][v] = (rw[j][0][v] ^ flip) >> (4 * fh);
            }
        }
        load_b(ks + 1, rw, rs);                       // (past the last step: loads nothing)
        const uint16_t *as = cur + (wm * TM + fr) * LDK + 8 * fh;
        // Each substep carries a share of the staging work (interleave + LDS store of the next
        // step's activations, loads two steps ahead) so it overlaps the MFMAs; the next
        // substep's A fragments are read before this substep's MFMAs.  Every wave finished
        // reading the other buffer before the barrier that ended the previous step.
        half8v a[2][FI];
#pragma unroll
        for (int i = 0; i < FI; ++i) a[0][i] = *reinterpret_cast<const half8v *>(as + 32 * i * LDK);
        // B operands one substep ahead: a substep's MFMAs depend on nothing computed in it, so
        // the next substep's sign expansion, A reads and staging run in their shadow
        // substep sub covers 16 k: binary word sub / 2, half sub % 2; ternary word sub
        auto expand = [&](int j, int sub) {
            if constexpr (T2) return expand_t2(nw[j][sub], s2[j]);
            else return (sub & 1) ? expand_pairs<8>(nw[j][sub >> 1], s2[j]) : expand_pairs<0>(nw[j][sub >> 1], s2[j]);
        };
        half8v b[2][FJ];
#pragma unroll
        for (int j = 0; j < FJ; ++j) b[0][j] = expand(j, 0);
#pragma unroll
        for (int sub = 0; sub < 8; ++sub) {           // 16 k per MFMA: word sub / 2, half sub % 2
            const int c = sub & 1;
#pragma unroll
            for (int i = 0; i < FI; ++i)
#pragma unroll
                for (int j = 0; j < FJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[c][i], b[c][j], acc[i][j], 0, 0, 0);
            if (sub < 7) {
#pragma unroll
                for (int i = 0; i < FI; ++i)
                    a[c ^ 1][i] = *reinterpret_cast<const half8v *>(as + 32 * i * LDK + 16 * (sub + 1));
#pragma unroll
                for (int j = 0; j < FJ; ++j) b[c ^ 1][j] = expand(j, sub + 1);
            }
#pragma unroll
            for (int i = sub; i < kAUnits; i += 8) {
                store_a1(nxt, i, ra[i]);
                load_a1(ks + 2, i, ra[i]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
    };
    // (an odd step count runs one extra step on all-zero operands, which adds exactly 0)
    for (int ks = 0; ks < nk; ks += 2) {
        step(ks, std::integral_constant<int, 0>{});
        step(ks + 1, std::integral_constant<int, 1>{});
    }

    // D layout of a 32x32 tile: lane l, value v -> row 8*(v/4) + 4*(l/32) + v%4, column l%32
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + wm * TM + 32 * i + 8 * (v >> 2) + 4 * fh + (v & 3);
                const int n = n0 + wn * TN + 32 * j + fr;
                if (m < M && n < N) y[(size_t)m * N + n] = f2h_rne(acc[i][j][v]);
            }
}

namespace {
template <int BM, int WM, int WN, int WPE, bool T2>
hipError_t launch_prefill_t(const uint16_t *x, const uint32_t *W, const uint16_t *S, uint16_t *y, int M, int K,
                            int N, hipStream_t st, std::string *desc)
{
    constexpr int shm = 2 * BM * LDK * 2;
    if (desc) {                                        // describe the launch instead of making it
        char buf[96];
        snprintf(buf, sizeof buf, "prefill<%d,%d,%d,%d,%d> grid=%d", BM, WM, WN, WPE, (int)T2,
                 ((M + BM - 1) / BM) * ((N + BN - 1) / BN));
        desc->append(desc->empty() ? "" : ";").append(buf);
        return hipSuccess;
    }
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&prefill_kernel<BM, WM, WN, WPE, T2>), hipFuncAttributeMaxDynamicSharedMemorySize,
        shm);
    if (attr != hipSuccess) return attr;
    const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    hipLaunchKernelGGL((prefill_kernel<BM, WM, WN, WPE, T2>), dim3(tm * tn), dim3(64 * WM * WN), shm, st, x, W, S, y,
                       M, K, N, tm);
    return hipGetLastError();
}
}  // namespace

// Four waves of 128 x 96 on 256 x 192 tiles, one wave per SIMD: measured fastest of the 4- and
// 8-wave layouts when the tiles fill the GPU twice over (the expansion and staging VALU work does
// not overlap the MFMAs of a second wave).  With fewer tiles than that (M <= 1024 at N = 12288)
// 128 x 192 tiles with two workgroups per CU keep every CU busy (M = 512: 59-63 us against
// 81-84 us).
static bool prefill_small_tiles(int M, int N) { return (long long)((M + 255) / 256) * ((N + 191) / 192) < 512; }

hipError_t launch_prefill(const uint16_t *x, const uint32_t *W, const uint16_t *S, uint16_t *y,
                          int M, int K, int N, hipStream_t st, std::string *desc)
{
    if (prefill_small_tiles(M, N)) return launch_prefill_t<128, 2, 2, 2, false>(x, W, S, y, M, K, N, st, desc);
    return launch_prefill_t<256, 2, 2, 1, false>(x, W, S, y, M, K, N, st, desc);
}

hipError_t launch_prefill_t2(const uint16_t *x, const uint32_t *T, const uint16_t *S, uint16_t *y,
                             int M, int K, int N, hipStream_t st, std::string *desc)
{
    if (prefill_small_tiles(M, N)) return launch_prefill_t<128, 2, 2, 2, true>(x, T, S, y, M, K, N, st, desc);
    return launch_prefill_t<256, 2, 2, 1, true>(x, T, S, y, M, K, N, st, desc);
}

}  // namespace bin1
