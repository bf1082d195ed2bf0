// noalloc.hip -- bin1_gemv_noalloc: the product of bin1_gemv_ws with the library's own scratch
// array instead of a caller's workspace, for callers that cannot allocate device memory (code
// under graph capture, serving loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ variable: every GPU the library runs on holds one copy
// until the process ends.  Its device address is looked up once per device, on that device's
// first call, and kept; host code never passes the array's own name (a host-side stand-in) to a
// kernel.  All calls on one GPU share that GPU's copy: calls that overlap in time on one GPU race.
// The split-K partial sums stored there are written in full before they are read, so nothing
// has to be cleared between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "bin1.h"
#include "kernels.hpp"

namespace {

constexpr size_t kScratchBytes = 4u << 20;          // 4 MiB per device
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];                        // device address of each GPU's copy

}  // namespace

extern "C" {

int bin1_gemv_noalloc(const void *x, const uint32_t *Wbits, const void *scales, void *y, int M, int K, int N,
                      void *stream)
{
    if (M >= 1 && N >= 1 && K >= 128 && K % 128 == 0 && bin1_gemv_workspace_bytes(M, K, N) > kScratchBytes)
        return bin1::set_error(BIN1_ERR_SHAPE, "bin1_gemv_noalloc: this shape needs more scratch than the "
                                               "library's 4 MiB (use bin1_gemv_ws)");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return bin1::set_error(BIN1_ERR_DEVICE, "bin1_gemv_noalloc: no usable current HIP device");
    void *ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        if (!g_scratch[dev]) {
            void *p = nullptr;
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) {
                (void)hipGetLastError();
                return bin1::set_error(BIN1_ERR_DEVICE, "bin1_gemv_noalloc: cannot resolve the scratch array's "
                                                        "device address");
            }
            g_scratch[dev] = p;
        }
        ptr = g_scratch[dev];
    }
    return bin1::gemv_scratch("bin1_gemv_noalloc", x, Wbits, scales, y, M, K, N, ptr, kScratchBytes, false, stream);
}

}  // extern "C"
