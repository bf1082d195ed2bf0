// prefill.hip -- prefill product y = x * W^T on the matrix cores.
//
// Prompt processing is compute-bound rather than bandwidth-bound ["Bonsai 27B" page,
// section "Low-bit kernels for hybrid attention"], so this is the one dense contraction:
// sign bits become fp16 +-scale operands (w = s_g * b, "Binary weight format" section,
// eq. b_eff) and are multiplied on the MFMA units with fp32 accumulation.  fp16 operands
// hold x and +-s exactly; bf16 would round both and runs at the same dense rate on gfx950.
//
// Tiling for gfx950: a 128 x 192 output tile per workgroup, two workgroups per CU (M=2048,
// N=12288 gives 1024 workgroups, two full rounds over 256 CUs); four waves side by side along N,
// each 128 x 48 as an 8 x 3 grid of v_mfma_f32_16x16x32_f16 accumulators (96 registers).  K
// advances 128 (one scale group) per step, in four 32-wide substeps.
//
//  * Activations go through LDS (two buffers, one barrier per step), in natural k order: the
//    next step's activations are loaded straight into the other buffer (buffer_load ... lds,
//    no registers and no LDS stores) while the MFMAs read the current one.
//  * Weights never touch LDS: every wave expands the bits of its own 48 columns straight into
//    B-operand registers, so each weight column is expanded exactly once per workgroup and each
//    expanded operand serves all 8 row blocks of the tile (two VALU operations per fp16 pair
//    per 128 rows).  A packed 16-bit shift of the half-word holding a lane's bits (read by both
//    halves) puts adjacent bits on bits 15 and 31, so an operand dword pairs consecutive k and
//    the staged activations need no permute; one and-or then lays both signs over |s| (a
//    negative scale is folded into the sign bits first).  Each lane takes its k-slots from two
//    words of a step (binary) or four contiguous words (ternary), so it loads 8 or 16 bytes of a
//    row per step.
//  * Workgroup b takes M-tile b % tiles_m: with 16 M-tiles each XCD keeps two activation
//    panels in its L2.
#include "common.hpp"
#include "kernels.hpp"

#include <cstdio>
#include <string>
#include <type_traits>

namespace bin1 {

namespace {

typedef unsigned u4v __attribute__((ext_vector_type(4)));
typedef unsigned u2v __attribute__((ext_vector_type(2)));
typedef unsigned short us2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int BN = 192, BK = 128;
constexpr int LDK = BK + 16;                      // LDS row stride in halves (288 B)
constexpr int kRsrcFlags = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcFlags);
}

// B-operand dword p of a lane (binary): fp16 pair (+-|s| for bit B + 2p, +-|s| for bit B + 2p + 1)
// of nw, where bit 1 of nw means a negative product and B is 0 or 16.  One packed 16-bit
// shift of the 16-bit half holding those bits (read by both halves) puts the pair on bits 15 and
// 31; one and-or keeps those two sign bits over |s| in both halves.
template <int B, int P>
__device__ __forceinline__ uint32_t expand_pair(uint32_t nw, uint32_t s2abs)
{
    const us2v v = us2v((unsigned short)(B < 16 ? nw : nw >> 16));
    constexpr int b = B % 16 + 2 * P;
    const us2v sh{(unsigned short)(15 - b), (unsigned short)(14 - b)};
    return (__builtin_bit_cast(uint32_t, v << sh) & 0x80008000u) | s2abs;
}

template <int B>
__device__ __forceinline__ half8v expand_b1(uint32_t nw, uint32_t s2abs)
{
    const u4v d{expand_pair<B, 0>(nw, s2abs), expand_pair<B, 1>(nw, s2abs), expand_pair<B, 2>(nw, s2abs),
                expand_pair<B, 3>(nw, s2abs)};
    return __builtin_bit_cast(half8v, d);
}

// Ternary (2-bit slots: low bit nonzero, high bit negative): dword p holds slots 2p and 2p + 1
// of the 8-slot chunk in the low 16 bits of nw.  Packed shifts put the two negative bits
// (4p + 1, 4p + 3) on bits 15 and 31 and the two nonzero bits (4p, 4p + 2) on bits 0 and 16;
// one 24-bit multiply by |s| turns the nonzero bits into |s| or 0 in each half.
template <int P>
__device__ __forceinline__ uint32_t expand_t2_pair(uint32_t nw, uint32_t sabs)
{
    const us2v v = us2v((unsigned short)nw);
    const us2v sh_sign{(unsigned short)(14 - 4 * P), (unsigned short)(12 - 4 * P)};
    const us2v sh_nz{(unsigned short)(4 * P), (unsigned short)(4 * P + 2)};
    const uint32_t sign = __builtin_bit_cast(uint32_t, v << sh_sign) & 0x80008000u;
    const uint32_t nz = __builtin_bit_cast(uint32_t, v >> sh_nz) & 0x00010001u;
    return sign | mul24(nz, sabs);
}

__device__ __forceinline__ half8v expand_t2(uint32_t nw, uint32_t sabs)
{
    const u4v d{expand_t2_pair<0>(nw, sabs), expand_t2_pair<1>(nw, sabs), expand_t2_pair<2>(nw, sabs),
                expand_t2_pair<3>(nw, sabs)};
    return __builtin_bit_cast(half8v, d);
}

}  // namespace

// BM x 192 tile; four waves side by side along N, each BM x 48 as FI x 3 fragments of
// v_mfma_f32_16x16x32_f16 (FI = BM / 16).  Every weight column of the tile is expanded by exactly
// one wave, and each expanded B operand feeds FI MFMAs.  WPE waves per SIMD (from one or several
// workgroups per CU).  T2: ternary weights in 2-bit slots (16 per word) instead of sign bits.
template <int BM, int WPE, bool T2>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void prefill_kernel(const uint16_t *__restrict__ x, const uint32_t *__restrict__ W,
                    const uint16_t *__restrict__ S, uint16_t *__restrict__ y, int M, int K, int N,
                    int tiles_m)
{
    constexpr int TN = BN / 4;
    constexpr int FI = BM / 16, FJ = TN / 16;
    constexpr int BUF_HALVES = BM * LDK;          // one activation buffer
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int t = threadIdx.x, lane = t & 63;
    const int wn = __builtin_amdgcn_readfirstlane(t >> 6);
    const int bm = blockIdx.x % tiles_m, bn = blockIdx.x / tiles_m;
    const int m0 = bm * BM, n0 = bn * BN;
    const int wpr = T2 ? K >> 4 : K >> 5, spr = K >> 7, nk = K / BK;
    // MFMA operand lanes: lane (c, g) holds row / column c of its fragment and MFMA k-slots
    // 8g .. 8g + 7.  In substep sub those slots take k = 64(g / 2) + 16 sub + 8(g % 2) + e (A and
    // B follow the same map, so the sum over k is unchanged).  A lane then needs two words of a
    // step (binary: bits 8(g % 2) .. of words 2(g / 2) and 2(g / 2) + 1) or four (ternary: slots
    // 8(g % 2) .. of words 4(g / 2) .. 4(g / 2) + 3), one load; and the two lane groups of a
    // half-wave read A at k offsets 8 apart, which at the 144-half row stride conflict on half as
    // many LDS banks as other offsets or strides tried.
    const int fc = lane & 15, fg = lane >> 4;
    const int ak = 64 * (fg >> 1) + 8 * (fg & 1);     // this lane's first k of substep 0
    constexpr int kSubK = 16;                          // k advance of a lane per substep

    const __amdgpu_buffer_rsrc_t rx = rsrc(x, (unsigned)M * (unsigned)K * 2u);
    const __amdgpu_buffer_rsrc_t rW = rsrc(W, (unsigned)N * (unsigned)wpr * 4u);
    const __amdgpu_buffer_rsrc_t rS = rsrc(S, (unsigned)N * (unsigned)spr * 2u);

    // ---- activation staging: straight from memory into LDS (`buffer_load_dwordx4 ... lds`, no
    // registers, no LDS stores).  One such load writes 64 consecutive 16-byte slots of the padded
    // LDS image of a step (row r, slot q at 16 (18 r + q) bytes; slots 16 and 17 of a row are
    // padding), lane l the l-th slot.  Wave w issues loads w kDma .. w kDma + kDma - 1 of a
    // step's kDma * 4.  A lane's global offset is fixed per load and the step's offset is a
    // uniform add, so the loads cost no VALU work; padding slots and rows past M point at the end
    // of x (out of range: zeros), and past the last step a uniform 2^31 is added.
    constexpr int kRowSlots = LDK / 8;                 // 16-byte slots per LDS row (16 + 2 padding)
    constexpr int kDma = BM * kRowSlots / 64 / 4;      // loads per wave per step
    static_assert(BM * kRowSlots % 256 == 0, "the padded image is a whole number of loads per wave");
    const unsigned xbytes = (unsigned)M * (unsigned)K * 2u;
    unsigned a_vofs[kDma];
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
        const int slot = (wn * kDma + i) * 64 + lane, row = slot / kRowSlots, q = slot % kRowSlots;
        const int m = m0 + row;
        a_vofs[i] = (q < 16 && m < M) ? ((unsigned)m * (unsigned)K + 8u * (unsigned)q) * 2u : xbytes;
    }
    auto dma_a = [&](int ks, uint16_t *buf) {
        const unsigned so = ks < nk ? (unsigned)(ks * BK * 2) : 0x80000000u;
#pragma unroll
        for (int i = 0; i < kDma; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (__attribute__((address_space(3))) void *)(buf + (wn * kDma + i) * 512), 16, (int)a_vofs[i], (int)so, 0, 0);
    };
    // ---- weight bits of this wave's FJ column fragments: row n0 + TN wn + 16 j + fc, this lane's
    // two words (ternary: four words) of a step and the group scale.  Rows past N lie past the
    // buffer's range and load zeros; past the last step a uniform 2^31 is added to every offset
    // (no per-lane select, which the compiler would turn into a branch around each load).
    unsigned b_wofs[FJ], b_sofs[FJ];                   // byte offsets of this lane's rows at step 0
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
        const unsigned n = (unsigned)(n0 + wn * TN + 16 * j + fc);
        b_wofs[j] = n * (unsigned)wpr * 4u + (T2 ? 16u : 8u) * (unsigned)(fg >> 1);
        b_sofs[j] = n * (unsigned)spr * 2u;
    }
    using WordT = std::conditional_t<T2, u4v, u2v>;
    auto load_b = [&](int ks, WordT (&rw)[FJ], uint32_t (&rs)[FJ]) {
        const unsigned sw = ks < nk ? (unsigned)((T2 ? 32 : 16) * ks) : 0x80000000u;
        const unsigned ss = ks < nk ? (unsigned)(2 * ks) : 0x80000000u;
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            if constexpr (T2) rw[j] = __builtin_amdgcn_raw_buffer_load_b128(rW, b_wofs[j] + sw, 0, 0);
            else rw[j] = __builtin_amdgcn_raw_buffer_load_b64(rW, b_wofs[j] + sw, 0, 0);
            rs[j] = __builtin_amdgcn_raw_buffer_load_b16(rS, b_sofs[j] + ss, 0, 0);
        }
    };

    f4v acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) acc[i][j] = f4v{0.f, 0.f, 0.f, 0.f};

    // Activations and weights are requested one K-step before use; the barrier that ends a step
    // waits for both (so the next step's activations are in LDS for every wave).  Loads are
    // unconditional (out-of-range offsets past the last step) so the loop is straight-line.
    WordT rw[FJ];
    uint32_t rs[FJ];
    dma_a(0, lds);
    load_b(0, rw, rs);
    __builtin_amdgcn_s_waitcnt(0x0F70);                // vmcnt(0): step 0's activations are in LDS
    __syncthreads();

    // one K-step on buffer P: the activations of step ks + 1 are requested into the other buffer
    // (every wave finished reading it before the barrier that ended the previous step), this
    // step's weights are folded and step ks + 1's requested in their place
    auto step = [&](int ks, auto P_c) {
        constexpr int P = decltype(P_c)::value;
        const uint16_t *cur = lds + P * BUF_HALVES;
        uint16_t *nxt = lds + (P ^ 1) * BUF_HALVES;
        dma_a(ks + 1, nxt);
        // this step's weights: fold each scale's sign into the bits and move this lane's eight
        // bits (ternary: slots) of each half-word to the bottom
        uint32_t nw[FJ][T2 ? 4 : 2], s2[FJ];
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            const uint32_t sv = rs[j] & 0xFFFFu;
            if constexpr (T2) {
                const uint32_t flip = (sv & 0x8000u) ? 0xAAAAAAAAu : 0u;   // negative scale: flip every slot's sign
                s2[j] = sv & 0x7FFFu;
#pragma unroll
                for (int sub = 0; sub < 4; ++sub) nw[j][sub] = (rw[j][sub] ^ flip) >> (16 * (fg & 1));
            } else {
                const uint32_t flip = (sv & 0x8000u) ? 0u : 0xFFFFFFFFu;   // bit 1 of nw: negative product
                s2[j] = (sv & 0x7FFFu) * 0x00010001u;
#pragma unroll
                for (int w = 0; w < 2; ++w) nw[j][w] = (rw[j][w] ^ flip) >> (8 * (fg & 1));
            }
        }
        load_b(ks + 1, rw, rs);                       // (past the last step: loads nothing)
        const uint16_t *as = cur + fc * LDK + ak;
        auto expand = [&](int j, auto sub_c) {
            constexpr int sub = decltype(sub_c)::value;
            if constexpr (T2) return expand_t2(nw[j][sub], s2[j]);
            else return expand_b1<16 * (sub & 1)>(nw[j][sub >> 1], s2[j]);
        };
        // A fragment r = FI sub + i is row block i of substep sub; it is read from LDS kAhead
        // fragments before its three MFMAs, so only kAhead + 1 fragments are live at a time.
        // A substep's B operands are expanded at its start (expanding them a substep ahead was
        // no faster).
        constexpr int kAhead = 8;
        auto read_a = [&](int r) { return *reinterpret_cast<const half8v *>(as + 16 * (r % FI) * LDK + kSubK * (r / FI)); };
        half8v a[4 * FI], b[FJ];
#pragma unroll
        for (int r = 0; r < kAhead; ++r) a[r] = read_a(r);
        auto substep = [&](auto sub_c) {              // 32 k per MFMA
            constexpr int sub = decltype(sub_c)::value;
#pragma unroll
            for (int j = 0; j < FJ; ++j) b[j] = expand(j, sub_c);
#pragma unroll
            for (int i = 0; i < FI; ++i) {
                const int r = FI * sub + i;
                if (r + kAhead < 4 * FI) a[r + kAhead] = read_a(r + kAhead);
#pragma unroll
                for (int j = 0; j < FJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[r], b[j], acc[i][j], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        substep(std::integral_constant<int, 0>{});
        substep(std::integral_constant<int, 1>{});
        substep(std::integral_constant<int, 2>{});
        substep(std::integral_constant<int, 3>{});
        // every load of this step (the next step's activations into LDS, its weights) has
        // landed before the barrier: s_waitcnt vmcnt(0), the other counters left alone
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    };
    // (an odd step count runs one extra step on all-zero operands, which adds exactly 0)
    for (int ks = 0; ks < nk; ks += 2) {
        step(ks, std::integral_constant<int, 0>{});
        step(ks + 1, std::integral_constant<int, 1>{});
    }

    // D layout of a 16x16 fragment: lane (c, g), value v -> row 4g + v, column c
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + 16 * i + 4 * fg + v;
                const int n = n0 + wn * TN + 16 * j + fc;
                if (m < M && n < N) y[(size_t)m * N + n] = f2h_rne(acc[i][j][v]);
            }
}

namespace {
template <int BM, int WPE, bool T2>
hipError_t launch_prefill_t(const uint16_t *x, const uint32_t *W, const uint16_t *S, uint16_t *y, int M, int K,
                            int N, hipStream_t st, std::string *desc)
{
    constexpr int shm = 2 * BM * LDK * 2;
    if (desc) {                                        // describe the launch instead of making it
        char buf[96];
        snprintf(buf, sizeof buf, "prefill<%d,%d,%d> grid=%d", BM, WPE, (int)T2,
                 ((M + BM - 1) / BM) * ((N + BN - 1) / BN));
        desc->append(desc->empty() ? "" : ";").append(buf);
        return hipSuccess;
    }
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&prefill_kernel<BM, WPE, T2>), hipFuncAttributeMaxDynamicSharedMemorySize, shm);
    if (attr != hipSuccess) return attr;
    const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    hipLaunchKernelGGL((prefill_kernel<BM, WPE, T2>), dim3(tm * tn), dim3(256), shm, st, x, W, S, y, M, K, N, tm);
    return hipGetLastError();
}
}  // namespace

// 128 x 192 tiles with two workgroups (two waves per SIMD) per CU, at every M.  At M = 2048,
// K = 4096, N = 12288 they measured 188-190 us against 200-202 us for 256 x 192 tiles with one
// workgroup per CU: with 256 rows a wave holds 192 accumulator and ~200 other registers, and
// the register allocator then shuttles staging data through AGPRs.
hipError_t launch_prefill(const uint16_t *x, const uint32_t *W, const uint16_t *S, uint16_t *y,
                          int M, int K, int N, hipStream_t st, std::string *desc)
{
    return launch_prefill_t<128, 2, false>(x, W, S, y, M, K, N, st, desc);
}

hipError_t launch_prefill_t2(const uint16_t *x, const uint32_t *T, const uint16_t *S, uint16_t *y,
                             int M, int K, int N, hipStream_t st, std::string *desc)
{
    return launch_prefill_t<128, 2, true>(x, T, S, y, M, K, N, st, desc);
}

}  // namespace bin1
