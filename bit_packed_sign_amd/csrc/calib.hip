// calib.hip -- two on-device references, neither doing any of the method's arithmetic:
//  * a plain streaming read of device memory: the HBM read rate that the decode kernels'
//    achieved bandwidth is compared against (every 16-byte chunk read once, folded into a digest
//    so that the loads cannot be dropped);
//  * a stream of independent fp16 matrix-core products: the MFMA rate this GPU sustains at the
//    clock it holds under such a load, which the prefill product is compared against.
#include "common.hpp"
#include "kernels.hpp"

namespace bin1 {

namespace {

typedef unsigned u4v __attribute__((ext_vector_type(4)));

// Thread t of T reads chunks t, t + T, t + 2T, ... (a wave reads 1 KiB contiguous per load
// instruction, the grid a contiguous T * 16 bytes per round), U loads in flight per thread.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u4v *__restrict__ p, size_t n16,
                                                          uint32_t *__restrict__ sink)
{
    const size_t T = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * T < n16; i += U * T) {
        u4v v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * T);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += T) {
        const u4v v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, kWave);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

// Every wave issues iters x 12 v_mfma_f32_32x32x16_f16 on 12 independent accumulators, nothing
// else inside the loop.  Lane l takes its A and B fragments (8 fp16 each) from ab[l] and ab[64 + l]:
// the operand values set how many multiplier bits toggle, and with them the power drawn and the
// clock the part holds.  Lane 0 of a wave writes the sum over the 12 accumulators of their element
// 0 (row 0, column 0 of the 32 x 32 product), 12 * iters * D00, to sink[global wave index].
__global__ __launch_bounds__(512) void mfma_rate_kernel(const half8v *__restrict__ ab, float *__restrict__ sink,
                                                        int iters)
{
    const int lane = threadIdx.x & 63;
    const half8v a = ab[lane], b = ab[64 + lane];
    f16v acc[12];
#pragma unroll
    for (int j = 0; j < 12; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 12; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 12; ++j) s += acc[j][0];
    if (lane == 0) sink[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = s;
}

}  // namespace

hipError_t launch_mfma_rate(const void *ab, float *sink, int grid, int waves, int iters, hipStream_t st)
{
    hipLaunchKernelGGL(mfma_rate_kernel, dim3(grid), dim3(64 * waves), 0, st, static_cast<const half8v *>(ab), sink,
                       iters);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, int grid, int unroll, hipStream_t st)
{
    const u4v *p = static_cast<const u4v *>(buf);
    const size_t n16 = bytes / 16;
    switch (unroll) {
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(grid), dim3(256), 0, st, p, n16, sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(grid), dim3(256), 0, st, p, n16, sink); break;
    default: hipLaunchKernelGGL(stream_read_kernel<16>, dim3(grid), dim3(256), 0, st, p, n16, sink); break;
    }
    return hipGetLastError();
}

}  // namespace bin1
