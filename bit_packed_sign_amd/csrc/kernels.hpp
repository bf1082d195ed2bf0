// kernels.hpp -- internal launchers behind the C ABI (include/bin1.h).  Each launcher
// assumes its arguments were validated by the API layer and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bin1 {

hipError_t launch_gemv(const uint16_t *x, const uint32_t *W, const uint16_t *S, uint16_t *y,
                       int M, int K, int N, hipStream_t st);
hipError_t launch_prefill(const uint16_t *x, const uint32_t *W, const uint16_t *S, uint16_t *y,
                          int M, int K, int N, hipStream_t st);
hipError_t launch_pm1(const uint32_t *A, const uint32_t *W, int32_t *y, int M, int K, int N,
                      hipStream_t st);
hipError_t launch_xor_patch(uint32_t *W, const int32_t *rows, int nrows, int K, int N,
                            int32_t *bad, hipStream_t st);
hipError_t launch_xor_patch_multi(uint32_t *const *Wtab, const int32_t *Ktab, const int32_t *Ntab,
                                  int nmat, const int32_t *entries, int nentries, int32_t *bad,
                                  hipStream_t st);

}  // namespace bin1
