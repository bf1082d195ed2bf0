// gemv_smallm.hip -- small-batch decode product (2 <= M <= 16 tokens) on fp16 MFMA.
//
// y[m][n] = sum_k s[n][k/128] * w(n,k) * x[m][k] ["Bonsai 27B" page, section "Binary weight
// format", eq. b_eff], fused decode with fp32 accumulation ["Bonsai 27B" page, section
// "Low-bit kernels for hybrid attention"].
//
// With M tokens each weight byte serves M products, so the per-weight expansion cost is
// amortised over the batch.  The tokens are the 16 A rows of v_mfma_f32_16x16x32_f16 (x is
// fp16 already, so A is exact; rows past M are zero).  The weight operand is built directly
// as fp16 +-|s| pairs: a pair takes one shift and one bit-field insert of the sign bit into
// |s| (the sign of a negative scale is folded into the word first), so the group scale is
// applied inside the product and the MFMA accumulates straight across groups.
#include "common.hpp"
#include "kernels.hpp"

namespace bin1 {

namespace {

typedef unsigned u4v __attribute__((ext_vector_type(4)));

constexpr int kRsrcFlags = 0x00020000;
constexpr unsigned kOob = 0x80000000u;
constexpr int kNT = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcFlags);
}

// fp16 +-|s| pairs for the 8 weights of byte `b` of word `nw` (nw: sign bit 1 = negative
// product).  Pair j holds the weights of bits 2j (low half) and 2j+1 (high half) of the byte,
// matching A's halves x[8b + 2j], x[8b + 2j + 1].  |s| has clear sign bits, so each pair is
// one shift and one and-or.
__device__ __forceinline__ half8 expand_byte(uint32_t nw, int b, uint32_t s2abs)
{
    const uint32_t by = (nw >> (8 * b)) & 0xFFu;
    const uint32_t tt = by | ((by >> 1) << 16);     // high copy pre-shifted by one bit
    uint32_t p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = ((tt << (15 - 2 * j)) & 0x80008000u) | s2abs;
    return __builtin_bit_cast(half8, u4v{p[0], p[1], p[2], p[3]});
}

constexpr int kWaves = 8;                            // waves per workgroup
constexpr int kChunkWords = 128;                     // 4096 weights per K chunk
constexpr int kWPW = kChunkWords / kWaves;           // words per wave in a chunk
constexpr int kGPW = kWPW / 4;                       // scale groups per wave in a chunk

// Work: a workgroup of 8 waves takes batches of up to TB 16-row tiles (grid-stride); for each
// batch it walks K in 4096-wide chunks.  In a chunk, wave w covers words [16w, 16w+16): its A
// operands (16 tokens x 512 k) are loaded into registers once per (batch, chunk) and reused
// by every tile of the batch.  Weights stream through a ring of P (chunk, tile) units.  The
// waves' partial tiles are merged through LDS at the end of each batch.
template <int P, int TB>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemv_smallm_kernel(const uint16_t *__restrict__ x, const uint32_t *__restrict__ W,
                        const uint16_t *__restrict__ S, uint16_t *__restrict__ y, int M, int K, int N,
                        int ntiles)
{
    __shared__ __attribute__((aligned(16))) float red[TB * 256 * kWaves];   // [tile][16 rows][16 tok][waves]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, b = lane >> 4;
    const int wpr = K >> 5, spr = K >> 7;
    const int nchunk = (wpr + kChunkWords - 1) / kChunkWords;
    const int my_tiles = blockIdx.x < ntiles ? (ntiles - 1 - blockIdx.x) / gridDim.x + 1 : 0;

    const __amdgpu_buffer_rsrc_t rx = rsrc(x, (unsigned)M * (unsigned)K * 2u);
    const __amdgpu_buffer_rsrc_t rW = rsrc(W, (unsigned)N * (unsigned)wpr * 4u);
    const __amdgpu_buffer_rsrc_t rS = rsrc(S, (unsigned)N * (unsigned)spr * 2u);

    u4v wb[P][kGPW];
    uint16_t sb[P][kGPW];
    // unit u of a batch = (chunk u / nb, tile u % nb); units past the batch load nothing
    auto issue = [&](int tb0, int nb, int u, u4v (&w)[kGPW], uint16_t (&s)[kGPW]) {
        const int c = u / nb, i = u - c * nb;
        const int row = (blockIdx.x + (tb0 + i) * gridDim.x) * 16 + n;
        const bool rok = c < nchunk && row < N;
#pragma unroll
        for (int q = 0; q < kGPW; ++q) {
            const int grp = (c * kChunkWords + wave * kWPW) / 4 + q;
            const bool ok = rok && grp < spr;
            w[q] = __builtin_amdgcn_raw_buffer_load_b128(rW, ok ? ((unsigned)row * wpr + 4u * grp) * 4u : kOob,
                                                        0, kNT);
            s[q] = __builtin_amdgcn_raw_buffer_load_b16(rS, ok ? ((unsigned)row * spr + grp) * 2u : kOob, 0, 0);
        }
    };

    for (int tb0 = 0; tb0 < my_tiles; tb0 += TB) {
        const int nb = my_tiles - tb0 < TB ? my_tiles - tb0 : TB;     // tiles in this batch
        const int nunits = nchunk * nb;
#pragma unroll
        for (int p = 0; p < P; ++p) issue(tb0, nb, p, wb[p], sb[p]);
        float4v acc[TB];
#pragma unroll
        for (int i = 0; i < TB; ++i) acc[i] = float4v{0.f, 0.f, 0.f, 0.f};
        half8 A[kWPW];
        for (int u0 = 0; u0 < nunits; u0 += P) {
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int u = u0 + p;
                if (u >= nunits) break;               // uniform
                const int c = u / nb, i = u - c * nb;
                if (i == 0) {                         // new chunk: this wave's A operands
#pragma unroll
                    for (int k = 0; k < kWPW; ++k) {
                        const int j = c * kChunkWords + wave * kWPW + k;   // word index
                        const bool ok = n < M && j < wpr;
                        const u4v v = __builtin_amdgcn_raw_buffer_load_b128(
                            rx, ok ? ((unsigned)n * K + 32u * j + 8u * b) * 2u : kOob, 0, 0);
                        A[k] = __builtin_bit_cast(half8, v);
                    }
                }
                float4v a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < kGPW; ++q) {
                    const uint32_t sbits = sb[p][q];
                    const uint32_t sabs = sbits & 0x7FFFu;
                    const uint32_t s2abs = sabs | (sabs << 16);
                    const uint32_t flip = (sbits & 0x8000u) ? 0u : 0xFFFFFFFFu;   // nw = w ^ flip
                    const u4v w = wb[p][q];
                    a = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[4 * q + 0], expand_byte(w.x ^ flip, b, s2abs), a, 0, 0, 0);
                    a = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[4 * q + 1], expand_byte(w.y ^ flip, b, s2abs), a, 0, 0, 0);
                    a = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[4 * q + 2], expand_byte(w.z ^ flip, b, s2abs), a, 0, 0, 0);
                    a = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[4 * q + 3], expand_byte(w.w ^ flip, b, s2abs), a, 0, 0, 0);
                }
                issue(tb0, nb, u + P, wb[p], sb[p]);
#pragma unroll
                for (int t = 0; t < TB; ++t)
                    if (t == i) acc[t] += a;
            }
        }
        // merge the four waves' K-slices; D layout: lane (n, b) holds tokens 4b..4b+3 of row n
        for (int t = 0; t < nb; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[((t * 16 + n) * 16 + 4 * b + r) * kWaves + wave] = acc[t][r];
        __syncthreads();
        for (int e = threadIdx.x; e < nb * 256; e += 64 * kWaves) {
            const int t = e >> 8, rr = (e >> 4) & 15, m = e & 15;
            const int row = (blockIdx.x + (tb0 + t) * gridDim.x) * 16 + rr;
            const float4v p0 = *reinterpret_cast<const float4v *>(red + (size_t)e * kWaves);
            const float4v p1 = *reinterpret_cast<const float4v *>(red + (size_t)e * kWaves + 4);
            const float tot = ((p0[0] + p0[1]) + (p0[2] + p0[3])) + ((p1[0] + p1[1]) + (p1[2] + p1[3]));
            if (m < M && row < N) y[(size_t)m * N + row] = f2h_rne(tot);
        }
        __syncthreads();
    }
}

template <int P, int TB>
hipError_t launch_sm(const uint16_t *x, const uint32_t *W, const uint16_t *S, uint16_t *y, int M, int K,
                     int N, hipStream_t st)
{
    const int tiles = (N + 15) / 16;
    const int grid = tiles < 256 ? tiles : 256;
    hipLaunchKernelGGL((gemv_smallm_kernel<P, TB>), dim3(grid), dim3(64 * kWaves), 0, st, x, W, S, y, M, K, N,
                       tiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_smallm(const uint16_t *x, const uint32_t *W, const uint16_t *S, uint16_t *y, int M,
                              int K, int N, hipStream_t st)
{
    return launch_sm<3, 4>(x, W, S, y, M, K, N, st);
}

}  // namespace bin1
