// pm1.hip -- +-1 activations times +-1 weights, exact in integers.
//
// With a, w in {-1,+1} held as bits (1 = +1), a*w = +1 exactly when the bits agree, so
// sum_k a_k w_k = K - 2 * popcount(a xor w): the product becomes bit operations
// ["PrismML Bonsai -- 1.15GB ..." page, section "What 1-bit is"].
#include "common.hpp"
#include "kernels.hpp"

namespace bin1 {

// LPR lanes per weight row (a power of two, at most the row's 16-byte chunks, at most 64), so a
// wave covers 64 / LPR rows at a time and no lane idles when a row is shorter than 1 KB (K = 4096:
// 32 chunks, two rows per wave); each wave takes R such row sets, whose loads go out together.
// Each lane xors/popcounts 16-byte chunks c, c + LPR, ... of its rows; MB activation rows share
// each weight load.  A row's lanes are reduced with xor-shuffles inside their group of LPR.
// Rows past N read row N - 1 (no branch around the loads) and store nothing.
template <int MB, int LPR, int R>
__global__ __launch_bounds__(256) void pm1_kernel(const uint32_t *__restrict__ A,
                                                  const uint32_t *__restrict__ W,
                                                  int32_t *__restrict__ y, int M, int K, int N)
{
    constexpr int RPW = 64 / LPR;                  // rows per wave and row set
    const int lane = threadIdx.x & 63;
    const int n0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW * R + lane / LPR;
    const int c0 = lane % LPR;
    const int q4 = K >> 7;                        // 16-byte chunks per row
    const uint4 *row[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int n = n0 + r * RPW;
        row[r] = reinterpret_cast<const uint4 *>(W + (size_t)(n < N ? n : N - 1) * (K >> 5));
    }
    for (int m0 = 0; m0 < M; m0 += MB) {
        int cnt[R][MB];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < MB; ++i) cnt[r][i] = 0;
        for (int c = c0; c < q4; c += LPR) {
            uint4 w[R];
#pragma unroll
            for (int r = 0; r < R; ++r) w[r] = row[r][c];
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                if (m0 + i < M) {
                    const uint4 a = reinterpret_cast<const uint4 *>(A + (size_t)(m0 + i) * (K >> 5))[c];
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        cnt[r][i] += __popc(a.x ^ w[r].x) + __popc(a.y ^ w[r].y) + __popc(a.z ^ w[r].z) +
                                     __popc(a.w ^ w[r].w);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = n0 + r * RPW;
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                int t = cnt[r][i];
#pragma unroll
                for (int off = LPR / 2; off >= 1; off >>= 1) t += __shfl_xor(t, off, kWave);
                if (c0 == 0 && n < N && m0 + i < M) y[(size_t)(m0 + i) * N + n] = K - 2 * t;
            }
        }
    }
}

template <int LPR>
hipError_t launch_pm1_l(const uint32_t *A, const uint32_t *W, int32_t *y, int M, int K, int N, hipStream_t st)
{
    // two row sets per wave: K = 4096, N = 151936 took 12.5-12.6 us against 15.1-15.3 with one
    // (and 12.7 with four), every result bit-exact
    constexpr int R = 2;
    constexpr int rows_per_wg = 4 * (64 / LPR) * R;
    dim3 grid((N + rows_per_wg - 1) / rows_per_wg), block(256);
    if (M == 1)
        hipLaunchKernelGGL((pm1_kernel<1, LPR, R>), grid, block, 0, st, A, W, y, M, K, N);
    else
        hipLaunchKernelGGL((pm1_kernel<8, LPR, R>), grid, block, 0, st, A, W, y, M, K, N);
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
