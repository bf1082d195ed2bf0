// gemv.hip -- decode GEMV y = x * W^T for 1-bit sign weights with fp16 group scales.
//
// Weight (n, k) = scales[n][k/128] * (bit (k%32) of Wbits[n][k/32] ? +1 : -1)
// ["Bonsai 27B" page, section "Binary weight format", eq. b_eff].  Signs are expanded
// by select/accumulate (no multiplies) and the group scale is applied once per 32-weight
// word partial sum; accumulation is fp32 ["Bonsai 27B" page, section "Low-bit kernels
// for hybrid attention"].
#include <string>

#include "common.hpp"
#include "kernels.hpp"

namespace bin1 {

// One wave per output row; lanes stride over the row's words.  MB activation rows are
// accumulated together so each weight word is read once per MB tokens.
template <int MB>
__global__ __launch_bounds__(256) void gemv_select_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ W, const uint16_t *__restrict__ S,
    uint16_t *__restrict__ y, int M, int K, int N)
{
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= N) return;
    const int wpr = K >> 5;
    const uint32_t *row = W + (size_t)n * wpr;
    const uint16_t *srow = S + (size_t)n * (K >> 7);
    for (int m0 = 0; m0 < M; m0 += MB) {
        float acc[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) acc[i] = 0.f;
        for (int j = lane; j < wpr; j += 64) {
            const uint32_t w = row[j];
            const float s = h2f(srow[j >> 2]);
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const int m = m0 + i;
                if (m < M) {
                    const uint4 *xp = reinterpret_cast<const uint4 *>(x + (size_t)m * K + 32 * j);
                    float p = 0.f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint4 v = xp[q];
                        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int h = 0; h < 8; ++h) {
                            const int b = q * 8 + h;
                            const float xv = h2f((uint16_t)(u[h >> 1] >> (16 * (h & 1))));
                            p += ((w >> b) & 1u) ? xv : -xv;
                        }
                    }
                    acc[i] += s * p;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const float t = wave_sum(acc[i]);
            if (lane == 0 && m0 + i < M) y[(size_t)(m0 + i) * N + n] = f2h_rne(t);
        }
    }
}

hipError_t launch_gemv(const uint16_t *x, const uint32_t *W, const uint16_t *S, uint16_t *y,
                       int M, int K, int N, hipStream_t st, std::string *desc)
{
    if (M > 16) return launch_prefill(x, W, S, y, M, K, N, st, desc);
    if (M == 1 && K <= mx_max_k()) {
        MxSet set{};
        set.W[0] = W; set.S[0] = S; set.y[0] = y; set.N[0] = N;
        set.tile_end[0] = (N + 15) / 16;
        set.count = 1;
        return launch_gemv_mx(x, set, K, st, desc);
    }
    if (M >= 2) {
        MxSet set{};
        set.W[0] = W; set.S[0] = S; set.y[0] = y; set.N[0] = N;
        set.count = 1;
        return launch_gemv_smallm(x, set, M, K, st, desc);
    }
    // M == 1 with K past the block-scaled kernel's register budget: select/accumulate
    dim3 grid((N + 3) / 4), block(256);
    if (desc) {                                        // describe the launch instead of making it
        desc->append(desc->empty() ? "" : ";").append("gemv_select<1> grid=" + std::to_string(grid.x));
        return hipSuccess;
    }
    hipLaunchKernelGGL(gemv_select_kernel<1>, grid, block, 0, st, x, W, S, y, M, K, N);
    return hipGetLastError();
}

}  // namespace bin1
