// patch.hip -- XOR row patch: complement every word of the listed output rows in place.
//
// A patch is a list of rows whose sign bits are all flipped; applying the same list
// again restores the weights ["LocalLLaMA ... XOR patch 'Bankai'" page, section "Key
// points"].  Flipping all K signs of row r negates y[:, r]; the scales are untouched.
#include "common.hpp"
#include "kernels.hpp"

namespace bin1 {

// One workgroup per patch entry; each thread complements 16-byte chunks of the row.
// Row bytes are K/8 = 16 * (K/128), so a row is a whole number of 16-byte chunks.
__global__ __launch_bounds__(64) void xor_patch_kernel(uint32_t *__restrict__ W,
                                                        const int32_t *__restrict__ rows,
                                                        int K, int N, int32_t *bad)
{
    const int r = rows[blockIdx.x];
    if (r < 0 || r >= N) {
        if (threadIdx.x == 0 && bad) atomicAdd(bad, 1);
        return;
    }
    const int chunks = K >> 7;
    uint4 *row = reinterpret_cast<uint4 *>(W + (size_t)r * (K >> 5));
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
        uint4 v = row[c];
        v.x = ~v.x; v.y = ~v.y; v.z = ~v.z; v.w = ~v.w;
        row[c] = v;
    }
}

__global__ __launch_bounds__(64) void xor_patch_multi_kernel(
    uint32_t *const *__restrict__ Wtab, const int32_t *__restrict__ Ktab,
    const int32_t *__restrict__ Ntab, int nmat, const int32_t *__restrict__ entries, int32_t *bad)
{
    const int id = entries[2 * blockIdx.x];
    const int r = entries[2 * blockIdx.x + 1];
    bool ok = id >= 0 && id < nmat;
    int K = 0;
    if (ok) {
        K = Ktab[id];
        ok = r >= 0 && r < Ntab[id] && K > 0 && (K & 127) == 0 && Wtab[id] != nullptr &&
             (reinterpret_cast<uintptr_t>(Wtab[id]) & 15u) == 0;
    }
    if (!ok) {
        if (threadIdx.x == 0 && bad) atomicAdd(bad, 1);
        return;
    }
    const int chunks = K >> 7;
    uint4 *row = reinterpret_cast<uint4 *>(Wtab[id] + (size_t)r * (K >> 5));
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
        uint4 v = row[c];
        v.x = ~v.x; v.y = ~v.y; v.z = ~v.z; v.w = ~v.w;
        row[c] = v;
    }
}

hipError_t launch_xor_patch(uint32_t *W, const int32_t *rows, int nrows, int K, int N,
                            int32_t *bad, hipStream_t st)
{
    hipLaunchKernelGGL(xor_patch_kernel, dim3(nrows), dim3(64), 0, st, W, rows, K, N, bad);
    return hipGetLastError();
}

hipError_t launch_xor_patch_multi(uint32_t *const *Wtab, const int32_t *Ktab, const int32_t *Ntab,
                                  int nmat, const int32_t *entries, int nentries, int32_t *bad,
                                  hipStream_t st)
{
    hipLaunchKernelGGL(xor_patch_multi_kernel, dim3(nentries), dim3(64), 0, st, Wtab, Ktab, Ntab,
                       nmat, entries, bad);
    return hipGetLastError();
}

}  // namespace bin1
