// calib.hip -- a plain streaming read of device memory: the HBM read rate that the decode
// kernels' achieved bandwidth is compared against.  It does none of the method's arithmetic;
// it only reads every 16-byte chunk once and folds the data into a digest so that the loads
// cannot be dropped.
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

}  // namespace

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
