// pm1.hip -- +-1 activations times +-1 weights, exact in integers.
//
// With a, w in {-1,+1} held as bits (1 = +1), a*w = +1 exactly when the bits agree, so
// sum_k a_k w_k = K - 2 * popcount(a xor w): the product becomes bit operations
// ["PrismML Bonsai -- 1.15GB ..." page, section "What 1-bit is"].
#include "common.hpp"
#include "kernels.hpp"

namespace bin1 {

// One wave per weight row; each lane xors/popcounts 4 words (16 B) per step, so a wave
// reads 1 KB of the row per load instruction.  MB activation rows share each weight load.
template <int MB>
__global__ __launch_bounds__(256) void pm1_kernel(const uint32_t *__restrict__ A,
                                                  const uint32_t *__restrict__ W,
                                                  int32_t *__restrict__ y, int M, int K, int N)
{
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= N) return;
    const int q4 = K >> 7;                        // 16-byte chunks per row
    const uint4 *row = reinterpret_cast<const uint4 *>(W + (size_t)n * (K >> 5));
    for (int m0 = 0; m0 < M; m0 += MB) {
        int cnt[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) cnt[i] = 0;
        for (int c = lane; c < q4; c += 64) {
            const uint4 w = row[c];
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                if (m0 + i < M) {
                    const uint4 a = reinterpret_cast<const uint4 *>(A + (size_t)(m0 + i) * (K >> 5))[c];
                    cnt[i] += __popc(a.x ^ w.x) + __popc(a.y ^ w.y) + __popc(a.z ^ w.z) +
                              __popc(a.w ^ w.w);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const int t = wave_sum_i(cnt[i]);
            if (lane == 0 && m0 + i < M) y[(size_t)(m0 + i) * N + n] = K - 2 * t;
        }
    }
}

hipError_t launch_pm1(const uint32_t *A, const uint32_t *W, int32_t *y, int M, int K, int N,
                      hipStream_t st)
{
    dim3 grid((N + 3) / 4), block(256);
    if (M == 1)
        hipLaunchKernelGGL(pm1_kernel<1>, grid, block, 0, st, A, W, y, M, K, N);
    else
        hipLaunchKernelGGL(pm1_kernel<8>, grid, block, 0, st, A, W, y, M, K, N);
    return hipGetLastError();
}

}  // namespace bin1
