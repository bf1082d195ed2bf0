// patch.hip -- XOR patches (whole rows, or single bits) and the scale ranking of rows.
//
// A patch is a list of rows whose sign bits are all flipped; applying the same list
// again restores the weights ["LocalLLaMA ... XOR patch 'Bankai'" page, section "Key
// points"].  Flipping all K signs of row r negates y[:, r]; the scales are untouched.
#include "common.hpp"
#include "kernels.hpp"

namespace bin1 {

// One workgroup per patch entry; each thread complements 8-byte words of the row with atomic
// XORs (no value returned, so they are issued and not waited on).  Complementing is an XOR, so
// entries commute: a row listed an even number of times in one call ends unchanged and an odd
// number of times complemented, whatever the order the workgroups run in.
__device__ __forceinline__ void complement_row(uint32_t *row32, int K)
{
    unsigned long long *row = reinterpret_cast<unsigned long long *>(row32);
    const int words = K >> 6;                              // K / 64 eight-byte words
    for (int c = threadIdx.x; c < words; c += blockDim.x) atomicXor(row + c, ~0ull);
}

__global__ __launch_bounds__(64) void xor_patch_kernel(uint32_t *__restrict__ W,
                                                        const int32_t *__restrict__ rows,
                                                        int K, int N, int32_t *bad)
{
    const int r = rows[blockIdx.x];
    if (r < 0 || r >= N) {
        if (threadIdx.x == 0 && bad) atomicAdd(bad, 1);
        return;
    }
    complement_row(W + (size_t)r * (K >> 5), K);
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
    complement_row(Wtab[id] + (size_t)r * (K >> 5), K);
}

// Bit-granular patch ["LocalLLaMA ... XOR patch 'Bankai'" page, experiments section: random
// flips of single MLP weight bits]: one thread per (matrix id, row, k) entry flips the sign bit
// of weight k.  Entries may repeat, so each flip is an atomic XOR on its word: flips commute,
// a bit listed twice is unchanged, and the same list applied again removes the patch.
__global__ __launch_bounds__(256) void xor_bits_kernel(uint32_t *const *__restrict__ Wtab,
                                                        const int32_t *__restrict__ Ktab,
                                                        const int32_t *__restrict__ Ntab, int nmat,
                                                        const int32_t *__restrict__ entries, int n, int32_t *bad)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int id = entries[3 * i], r = entries[3 * i + 1], k = entries[3 * i + 2];
    uint32_t *W = nullptr;
    int K = 0;
    bool ok = id >= 0 && id < nmat;
    if (ok) {
        K = Ktab[id];
        W = Wtab[id];
        ok = K > 0 && (K & 127) == 0 && r >= 0 && r < Ntab[id] && k >= 0 && k < K && W != nullptr &&
             (reinterpret_cast<uintptr_t>(W) & 15u) == 0;
    }
    if (!ok) {
        if (bad) atomicAdd(bad, 1);
        return;
    }
    atomicXor(W + (size_t)r * (unsigned)(K >> 5) + (k >> 5), 1u << (k & 31));
}

// Scale ranking of rows [same page: targeting by scale factors].  Score of row n: the sum of
// its |scale| in units of 2^-24 (the smallest fp16 subnormal), an exact integer: a magnitude
// with biased exponent e and fraction f is f units when e = 0, else (f + 2^10) << (e - 1).
__global__ __launch_bounds__(256) void row_score_kernel(const uint16_t *__restrict__ S, int N, int groups,
                                                         int64_t *__restrict__ score)
{
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    const uint16_t *row = S + (size_t)n * groups;
    int64_t acc = 0;
    for (int g = 0; g < groups; ++g) {
        const uint32_t h = row[g] & 0x7FFFu;
        const uint32_t e = h >> 10;
        const int64_t mant = e ? (int64_t)((h & 0x3FFu) | 0x400u) : (int64_t)h;
        acc += mant << (e ? e - 1 : 0);
    }
    score[n] = acc;
}

// order[rank(n)] = n, rank(n) = number of rows m ahead of n: score[m] > score[n], or equal
// scores and m < n.  (row, score) pairs are distinct, so the ranks are a permutation.  Each
// thread counts over all rows, staged 1024 at a time through LDS: O(N^2), for N <= 2^20.
__global__ __launch_bounds__(256) void rank_rows_kernel(const int64_t *__restrict__ score, int N,
                                                         int32_t *__restrict__ order)
{
    __shared__ int64_t tile[1024];
    const int n = blockIdx.x * 256 + threadIdx.x;
    const int64_t me = n < N ? score[n] : 0;
    int rank = 0;
    for (int base = 0; base < N; base += 1024) {
        __syncthreads();
        for (int j = threadIdx.x; j < 1024; j += 256) tile[j] = base + j < N ? score[base + j] : 0;
        __syncthreads();
        const int lim = N - base < 1024 ? N - base : 1024;
        for (int j = 0; j < lim; ++j) {
            const int64_t v = tile[j];
            rank += (v > me) | ((v == me) & (base + j < n));
        }
    }
    if (n < N) order[rank] = n;
}

hipError_t launch_xor_bits(uint32_t *const *Wtab, const int32_t *Ktab, const int32_t *Ntab, int nmat,
                           const int32_t *entries, int n, int32_t *bad, hipStream_t st)
{
    hipLaunchKernelGGL(xor_bits_kernel, dim3((n + 255) / 256), dim3(256), 0, st, Wtab, Ktab, Ntab, nmat, entries, n,
                       bad);
    return hipGetLastError();
}

hipError_t launch_rank_rows(const uint16_t *S, int N, int K, int64_t *score, int32_t *order, hipStream_t st)
{
    hipLaunchKernelGGL(row_score_kernel, dim3((N + 255) / 256), dim3(256), 0, st, S, N, K >> 7, score);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(rank_rows_kernel, dim3((N + 255) / 256), dim3(256), 0, st, score, N, order);
    return hipGetLastError();
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
