// prefill.hip -- prefill product y = x * W^T on the matrix cores.
//
// Prompt processing is compute-bound rather than bandwidth-bound ["Bonsai 27B" page,
// section "Low-bit kernels for hybrid attention"], so this is the one dense contraction:
// each K-tile of sign bits is unpacked into LDS as fp16 +-scale (w = s_g * b, "Binary
// weight format" section, eq. b_eff) and multiplied on the MFMA units with fp32
// accumulation.  fp16 operands hold x and +-s exactly; bf16 would round both and runs at
// the same dense rate on gfx950.
#include "common.hpp"
#include "kernels.hpp"

namespace bin1 {

namespace {
constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8;   // LDS row stride in halves (144 B)
}

__global__ __launch_bounds__(256) void prefill_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ W, const uint16_t *__restrict__ S,
    uint16_t *__restrict__ y, int M, int K, int N)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDK];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int wpr = K >> 5, spr = K >> 7;

    float4v acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};

    const int lr = t >> 1, part = t & 1;     // loader: tile row, 32-wide half of the K-tile

    for (int k0 = 0; k0 < K; k0 += BK) {
        // activations: 32 halves (64 B) per thread
        {
            uint4 v[4];
            const int m = m0 + lr;
            if (m < M) {
                const uint4 *src = reinterpret_cast<const uint4 *>(x + (size_t)m * K + k0 + 32 * part);
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = src[q];
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = uint4{0, 0, 0, 0};
            }
            uint4 *dst = reinterpret_cast<uint4 *>(As + lr * LDK + 32 * part);
#pragma unroll
            for (int q = 0; q < 4; ++q) dst[q] = v[q];
        }
        // weights: one 32-bit word -> 32 fp16 values +-s
        {
            uint4 v[4];
            const int n = n0 + lr;
            if (n < N) {
                const uint32_t w = W[(size_t)n * wpr + (k0 >> 5) + part];
                const uint32_t sb = S[(size_t)n * spr + (k0 >> 7)];
                const uint32_t s2 = sb | (sb << 16);
                const uint32_t nw = ~w;                     // bit 0 -> negative weight
                uint32_t u[16];
#pragma unroll
                for (int p = 0; p < 16; ++p) {
                    const uint32_t lo = (nw >> (2 * p)) & 1u, hi = (nw >> (2 * p + 1)) & 1u;
                    u[p] = s2 ^ ((lo << 15) | (hi << 31));
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = uint4{u[4 * q], u[4 * q + 1], u[4 * q + 2], u[4 * q + 3]};
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = uint4{0, 0, 0, 0};
            }
            uint4 *dst = reinterpret_cast<uint4 *>(Bs + lr * LDK + 32 * part);
#pragma unroll
            for (int q = 0; q < 4; ++q) dst[q] = v[q];
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            half8 a[4], b[4];
            const int kofs = kk + 8 * (lane >> 4);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *reinterpret_cast<const half8 *>(As + (wm * 64 + 16 * i + (lane & 15)) * LDK + kofs);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = *reinterpret_cast<const half8 *>(Bs + (wn * 64 + 16 * j + (lane & 15)) * LDK + kofs);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
    // D layout of a 16x16 tile: lane holds rows 4*(lane/16)+r, column lane%16.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 64 + 16 * i + 4 * (lane >> 4) + r;
                const int n = n0 + wn * 64 + 16 * j + (lane & 15);
                if (m < M && n < N) y[(size_t)m * N + n] = f2h_rne(acc[i][j][r]);
            }
}

hipError_t launch_prefill(const uint16_t *x, const uint32_t *W, const uint16_t *S, uint16_t *y,
                          int M, int K, int N, hipStream_t st)
{
    dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM), block(256);
    hipLaunchKernelGGL(prefill_kernel, grid, block, 0, st, x, W, S, y, M, K, N);
    return hipGetLastError();
}

}  // namespace bin1
