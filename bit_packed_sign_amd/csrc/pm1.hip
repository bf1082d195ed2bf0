// pm1.hip -- +-1 activations times +-1 weights, exact in integers.
//
// With a, w in {-1,+1} held as bits (1 = +1), a*w = +1 exactly when the bits agree, so
// sum_k a_k w_k = K - 2 * popcount(a xor w): the product becomes bit operations
// ["PrismML Bonsai -- 1.15GB ..." page, section "What 1-bit is"].
#include "common.hpp"
#include "kernels.hpp"

namespace bin1 {

// LPR lanes per weight row (a power of two, at most the row's 16-byte chunks, at most 64), so a
// wave covers 64 / LPR rows and no lane idles when a row is shorter than 1 KB (K = 4096: 32
// chunks, two rows per wave).  Each lane xors/popcounts 16-byte chunks c, c + LPR, ... of its row;
// MB activation rows share each weight load.  The row's lanes are reduced with xor-shuffles
// inside their group of LPR.
template <int MB, int LPR>
__global__ __launch_bounds__(256) void pm1_kernel(const uint32_t *__restrict__ A,
                                                  const uint32_t *__restrict__ W,
                                                  int32_t *__restrict__ y, int M, int K, int N)
{
    constexpr int RPW = 64 / LPR;                  // rows per wave
    const int lane = threadIdx.x & 63;
    const int n = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
    const int c0 = lane % LPR;
    const bool live = n < N;
    const int q4 = K >> 7;                        // 16-byte chunks per row
    const uint4 *row = reinterpret_cast<const uint4 *>(W + (size_t)(live ? n : 0) * (K >> 5));
    for (int m0 = 0; m0 < M; m0 += MB) {
        int cnt[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) cnt[i] = 0;
        for (int c = c0; c < q4 && live; c += LPR) {
            const uint4 w = row[c];
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                if (m0 + i < M) {
                    const uint4 a = reinterpret_cast<const uint4 *>(A + (size_t)(m0 + i) * (K >> 5))[c];
                    cnt[i] += __popc(a.x ^ w.x) + __popc(a.y ^ w.y) + __popc(a.z ^ w.z) + __popc(a.w ^ w.w);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            int t = cnt[i];
#pragma unroll
            for (int off = LPR / 2; off >= 1; off >>= 1) t += __shfl_xor(t, off, kWave);
            if (c0 == 0 && live && m0 + i < M) y[(size_t)(m0 + i) * N + n] = K - 2 * t;
        }
    }
}

template <int LPR>
hipError_t launch_pm1_l(const uint32_t *A, const uint32_t *W, int32_t *y, int M, int K, int N, hipStream_t st)
{
    constexpr int rows_per_wg = 4 * (64 / LPR);
    dim3 grid((N + rows_per_wg - 1) / rows_per_wg), block(256);
    if (M == 1)
        hipLaunchKernelGGL((pm1_kernel<1, LPR>), grid, block, 0, st, A, W, y, M, K, N);
    else
        hipLaunchKernelGGL((pm1_kernel<8, LPR>), grid, block, 0, st, A, W, y, M, K, N);
    return hipGetLastError();
}

hipError_t launch_pm1(const uint32_t *A, const uint32_t *W, int32_t *y, int M, int K, int N,
                      hipStream_t st)
{
    const int chunks = K >> 7;                    // >= 1
    if (chunks >= 64) return launch_pm1_l<64>(A, W, y, M, K, N, st);
    if (chunks >= 32) return launch_pm1_l<32>(A, W, y, M, K, N, st);
    if (chunks >= 16) return launch_pm1_l<16>(A, W, y, M, K, N, st);
    if (chunks >= 8) return launch_pm1_l<8>(A, W, y, M, K, N, st);
    if (chunks >= 4) return launch_pm1_l<4>(A, W, y, M, K, N, st);
    if (chunks >= 2) return launch_pm1_l<2>(A, W, y, M, K, N, st);
    return launch_pm1_l<1>(A, W, y, M, K, N, st);
}

}  // namespace bin1
