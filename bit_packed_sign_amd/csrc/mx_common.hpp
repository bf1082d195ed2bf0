// mx_common.hpp -- pieces shared by the block-scaled (fp4 x fp8) MFMA decode kernels.
//
// Weights: one packed word (32 signs, bit 1 = +1) becomes 32 fp4 e2m1 values +-1 (the
// multiply-free sign expansion of the "PrismML Bonsai -- 1.15GB" page, section "What 1-bit
// is"); activations: each 32-element block of x becomes e4m3 limbs with per-block E8M0
// exponents.  v_mfma_scale_f32_16x16x128_f8f6f4 contracts them, one 128-weight group per
// chain of four instructions ("Bonsai 27B" page, section "Binary weight format", eq. b_eff).
#pragma once

#include "common.hpp"

namespace bin1 {
namespace mx {

typedef unsigned u4v __attribute__((ext_vector_type(4)));

// Raw buffer resources: loads past num_records return 0 and stores past it are dropped,
// so ragged tiles and dead ring slots need no branches (branch-free code also lets the
// compiler count outstanding loads exactly, which keeps a prefetch ring full).
constexpr int kRsrcFlags = 0x00020000;
constexpr unsigned kOob = 0x80000000u;          // an offset past every resource
constexpr int kNT = 2;                           // cache policy: nontemporal (streamed once)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcFlags);
}

constexpr int kBlk = 528;          // LDS bytes per (segment, word): 16 rows x 32 B + 16 zero bytes
constexpr int kZero = 512;         // offset of the zero bytes inside a block

// fp4 (e2m1) expansion of one word: nibble q of register v = 0x2 | bit(4q+v) << 3,
// i.e. -1.0 for a set bit and +1.0 for a clear one (the sign is undone by the caller).
// Each register is one shift and one v_and_or_b32 (gfx9 encodes no literal in a three-operand
// instruction, and reads at most one scalar register: the mask comes from a scalar register, the
// +1.0 pattern from a vector one).
__device__ __forceinline__ int8v unpack_fp4(uint32_t w)
{
    const uint32_t sign = __builtin_amdgcn_readfirstlane(0x88888888u);
    const uint32_t one = 0x22222222u;
    int8v b;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(b[0]) : "v"(w << 3), "s"(sign), "v"(one));
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(b[1]) : "v"(w << 2), "s"(sign), "v"(one));
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(b[2]) : "v"(w << 1), "s"(sign), "v"(one));
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(b[3]) : "v"(w), "s"(sign), "v"(one));
    b[4] = b[5] = b[6] = b[7] = 0;
    return b;
}

// A operand of (segment, word t) for this lane, from a limb block in LDS.
__device__ __forceinline__ int8v load_a(const uint8_t *blk, int lo, int hi)
{
    const u4v a0 = *reinterpret_cast<const u4v *>(blk + lo);
    const u4v a1 = *reinterpret_cast<const u4v *>(blk + hi);
    int8v a;
    a[0] = a0.x; a[1] = a0.y; a[2] = a0.z; a[3] = a0.w;
    a[4] = a1.x; a[5] = a1.y; a[6] = a1.z; a[7] = a1.w;
    return a;
}

// fp4 (e2m1) expansion of two words of ternary 2-bit slots (low bit: nonzero, high bit:
// negative), 32 weights: the nibble's exponent bit 1 takes the slot's nonzero bit and its sign
// bit 3 the slot's negative bit, giving 0, +1.0 or -1.0 (code 10 gives -0).  Register 0 holds
// the even slots of wa, 1 its odd slots, 2 and 3 those of wb, so B element j is weight
// k(j) = 16 (j / 16) + 2 (j % 8) + (j / 8) % 2 of the 32.
__device__ __forceinline__ int8v unpack_t2(uint32_t wa, uint32_t wb)
{
    int8v b;
    b[0] = (int)(((wa << 1) & 0x22222222u) | ((wa << 2) & 0x88888888u));
    b[1] = (int)(((wa >> 1) & 0x22222222u) | (wa & 0x88888888u));
    b[2] = (int)(((wb << 1) & 0x22222222u) | ((wb << 2) & 0x88888888u));
    b[3] = (int)(((wb >> 1) & 0x22222222u) | (wb & 0x88888888u));
    b[4] = b[5] = b[6] = b[7] = 0;
    return b;
}

template <int T>
__device__ __forceinline__ float4v mma_b(const int8v &a, const int8v &b, int scA, float4v c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, T, scA, 0, 127);
}

template <int T>
__device__ __forceinline__ float4v mma(const int8v &a, uint32_t w, int scA, float4v c)
{
    return mma_b<T>(a, unpack_fp4(w), scA, c);
}

// Lane offsets of the A operand inside a limb block: rows m = 4G + r of the MFMA are
// (group G, limb r) and are nonzero only in K-block G; lane (m, g) reads its 16-byte halves
// from row m or from the zero bytes.
__device__ __forceinline__ void a_offsets(int lane, int &lo, int &hi)
{
    const int m = lane & 15, g = lane >> 4, G = m >> 2;
    lo = (G == (g >> 1)) ? m * 32 + 16 * (g & 1) : kZero;
    hi = (G == 2 + (g >> 1)) ? m * 32 + 16 * (g & 1) : kZero;
}

// Limbs of 16 activations (one half h of a 32-element block) into a limb block.
// p0, p1: the 16 fp16 values; `mx` must already be the max |x| over the whole 32-block.
// blk: the block of (segment, word t); G: the block's MFMA K-block; scbyte: E8M0 bytes of
// rows 4G..4G+3 for word t (stride 4 bytes), written by the h == 0 half.
// Element j of a block row must pair with the weight the B operand puts there:
//  * binary (unpack_fp4): bit pi(j) = 4*(j%8) + j/8, so activation i of the half sits at byte
//    j = 8*(i%4) + 4h + i/4 -- dword 2c + h holds activations c, 4+c, 8+c, 12+c;
//  * ternary (unpack_t2): weight k(j) = 16 (j/16) + 2 (j%8) + (j/8)%2, so activation i sits at
//    byte 16h + 8 (i%2) + i/2 -- dword 4h + c holds activations 8m + e, 8m + 2 + e, 8m + 4 + e,
//    8m + 6 + e for c = 2e + m.
typedef _Float16 h2v __attribute__((ext_vector_type(2)));

template <bool T2 = false>
__device__ __forceinline__ void convert16(const u4v p0, const u4v p1, float mx, uint8_t *blk, int G, int h,
                                          uint8_t *scbyte)
{
    // activation of byte b of dword slot c
    auto idx = [](int c, int b) { return T2 ? 8 * (c & 1) + 2 * b + (c >> 1) : 4 * b + c; };
    const uint32_t hw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    const int e0 = mx > 0.f ? __builtin_amdgcn_frexp_expf(mx) - 1 : 0;   // 2^e0 <= mx
    if (e0 >= -4 && e0 <= 7) {
        // The same limbs in packed fp16, for blocks whose largest magnitude lies in [2^-4, 2^8):
        // there u = x 2^(7 - e0) scales x up (exact), and every value below is exact in fp16.
        //  * limb 0: the scaled conversion divides by its scale, fp8(x / 2^(e0 - 7)) = fp8(u),
        //    with the same rounding as the f32 conversion (checked over every fp16 value);
        //  * the next limb's input 16 (u - q): the back conversion multiplies by its scale (a
        //    power of two; its sign is not used), so scale 16 gives 16 q exactly, and one fma of x
        //    by 2^(11 - e0) <= 2^15 less that is 16 u - 16 q, exact (u - q carries at most 8
        //    significant bits).
        // Pairs are regrouped first so that each conversion fills the two bytes its dword holds.
        h2v P[4][2];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int i0 = idx(c, 2 * q), i1 = idx(c, 2 * q + 1);   // same parity
                P[c][q] = __builtin_bit_cast(h2v, __builtin_amdgcn_perm(hw[i1 >> 1], hw[i0 >> 1],
                                                                         (i0 & 1) ? 0x07060302u : 0x05040100u));
            }
        const float s0 = __builtin_ldexpf(1.0f, e0 - 7);
        const _Float16 f16 = (_Float16)__builtin_ldexpf(1.0f, 11 - e0);
        const h2v f16v = {f16, f16}, sixteen = {(_Float16)16.0f, (_Float16)16.0f};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int d[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (r < 3) {
                    const float sc = r == 0 ? s0 : 1.0f;
                    typedef short s2v __attribute__((ext_vector_type(2)));
                    s2v v = {0, 0};
                    v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(v, P[c][0], sc, false);
                    v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(v, P[c][1], sc, true);
                    d[c] = __builtin_bit_cast(int, v);
                } else {
                    d[c] = 0;
                }
                *reinterpret_cast<int *>(blk + (4 * G + r) * 32 + (T2 ? 4 * h + c : 2 * c + h) * 4) = d[c];
            }
            if (h == 0) scbyte[r * 4] = (uint8_t)(127 + e0 - 7 - 4 * r);
            if (r < 2) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const h2v m0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)d[c], 16.0f, false);
                    const h2v m1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)d[c], 16.0f, true);
                    P[c][0] = __builtin_elementwise_fma(P[c][0], r == 0 ? f16v : sixteen, -m0);
                    P[c][1] = __builtin_elementwise_fma(P[c][1], r == 0 ? f16v : sixteen, -m1);
                }
            }
        }
        return;
    }
    float u[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) u[i] = h2f((uint16_t)(hw[i >> 1] >> (16 * (i & 1))));
    const float mul = __builtin_ldexpf(1.0f, 7 - e0);
#pragma unroll
    for (int i = 0; i < 16; ++i) u[i] *= mul;        // |u| < 256, exact
    // Three limbs carry 12 significant bits, one more than fp16: every element within 2^10 of
    // the block's maximum is represented exactly, and no element is off by more than 2^-25 of
    // that maximum (e4m3's subnormals limit the smallest ones; checked over every fp16 value and
    // block exponent).  The fourth limb row of the A operand is stored as zeros, with a finite
    // exponent byte, so it contributes exactly 0.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        int d[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (r < 3) {
                int v = __builtin_amdgcn_cvt_pk_fp8_f32(u[idx(c, 0)], u[idx(c, 1)], 0, false);
                d[c] = __builtin_amdgcn_cvt_pk_fp8_f32(u[idx(c, 2)], u[idx(c, 3)], v, true);
            } else {
                d[c] = 0;
            }
            *reinterpret_cast<int *>(blk + (4 * G + r) * 32 + (T2 ? 4 * h + c : 2 * c + h) * 4) = d[c];
        }
        if (h == 0) scbyte[r * 4] = (uint8_t)(127 + e0 - 7 - 4 * r);
        if (r < 2) {
            // next limb's input: 16 (u - q), q = the fp8 value just stored.  u - q is exact
            // (q is u rounded to 4 significant bits) and so are 16 u and 16 q, so the single
            // fma 16 u - 16 q rounds nothing.
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                u[idx(c, 0)] = fmaf(u[idx(c, 0)], 16.f, -16.f * __builtin_amdgcn_cvt_f32_fp8(d[c], 0));
                u[idx(c, 1)] = fmaf(u[idx(c, 1)], 16.f, -16.f * __builtin_amdgcn_cvt_f32_fp8(d[c], 1));
                u[idx(c, 2)] = fmaf(u[idx(c, 2)], 16.f, -16.f * __builtin_amdgcn_cvt_f32_fp8(d[c], 2));
                u[idx(c, 3)] = fmaf(u[idx(c, 3)], 16.f, -16.f * __builtin_amdgcn_cvt_f32_fp8(d[c], 3));
            }
        }
    }
}

// max |x| over 16 fp16 values (packed fp16 max: exact, and a quarter of the scalar ops)
__device__ __forceinline__ float absmax16(const u4v p0, const u4v p1)
{
    const uint32_t hw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    h2v m[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = __builtin_elementwise_abs(__builtin_bit_cast(h2v, hw[i]));
#pragma unroll
    for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) m[i] = __builtin_elementwise_max(m[i], m[i + w]);
    return fmaxf((float)m[0].x, (float)m[0].y);
}

// Sum over the four lanes n, n+16, n+32, n+48 (every lane gets its column's total).
__device__ __forceinline__ float sum_groups(float v)
{
    const int iv = __builtin_bit_cast(int, v);
    const auto a = __builtin_amdgcn_permlane32_swap(iv, iv, false, false);
    v = __builtin_bit_cast(float, (int)a[0]) + __builtin_bit_cast(float, (int)a[1]);
    const int iw = __builtin_bit_cast(int, v);
    const auto b = __builtin_amdgcn_permlane16_swap(iw, iw, false, false);
    return __builtin_bit_cast(float, (int)b[0]) + __builtin_bit_cast(float, (int)b[1]);
}

}  // namespace mx
}  // namespace bin1
