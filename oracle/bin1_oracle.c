/*
 * bin1_oracle.c -- plain, slow, fp64 CPU oracle for the 1-bit sign GEMV, the
 * +-1 popcount product, the XOR row and bit patches and the scale ranking of rows.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link or call this
 * file; only the tests, the smoke check and the benchmark's CPU-baseline leg do.
 * It shares no source with the HIP library: the fp16 decode, bit indexing and
 * patch logic below are written out independently from their definitions.
 *
 * Sources (pages, by title and section):
 *  - "Bonsai 27B: ... (feat. PrismML)", discuss.pytorch.kr, section on the binary
 *    weight format (eq. b_eff): each weight is one sign bit in {-1,+1}; each
 *    group of 128 weights shares one fp16 scale, so w = s_g * b.
 *  - same page, section on the low-bit kernels: the fused kernel decodes the
 *    sign codes and applies the per-group fp16 scale inside the matmul, with
 *    activations and accumulation kept in high precision -- i.e. the result is
 *    the dequantise-and-dot, which is what this file computes, in fp64.
 *  - "PrismML Bonsai -- 1.15GB ..." (jangwook.net), section on what 1-bit means:
 *    with weights in {-1,+1} products become additions and subtractions, and the
 *    matmul becomes bit operations (the +-1 popcount mode).
 *  - "LocalLLaMA ... XOR patch 'Bankai'" (insights.marvin-42.com), key-points
 *    section: a patch is a list of (layer, projection, row) entries whose bits
 *    are flipped; the same XOR applies and removes it.
 *
 * Readings where the pages are silent:
 *  - bit order: bit b of word j is weight k = 32*j + b (LSB first); bit 1 = +1.
 *  - the scale group runs along K, aligned at k = 0; G is a parameter here only
 *    so that tiny cases (K < 128) can be enumerated exhaustively.
 *  - a patched "row" is one output row n: all of its K bits; scales untouched.
 *
 * Layouts (row-major, contiguous):
 *   x      fp16 bits [M][K]
 *   W      uint32    [N][ceil(K/32)]
 *   S      fp16 bits [N][K/G]
 *   y, nrm double    [M][N]
 */
#include <math.h>
#include <stdlib.h>
#include <stdint.h>
#include <omp.h>

/* IEEE 754 binary16 -> binary64, from the format definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 encodes
 * zero/subnormals (fraction * 2^-24), exponent 31 encodes inf/NaN. Exact. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -v : v;
}

/* Sign of weight (n, k): +1 if its bit is set, -1 otherwise. */
static inline double weight_sign(const uint32_t *row, int64_t k)
{
    uint32_t word = row[k / 32];
    return ((word >> (k % 32)) & 1u) ? 1.0 : -1.0;
}

/* y[m][n]   = sum_k S[n][k/G] * w(n,k) * x[m][k]   (ascending k, fp64)
 * nrm[m][n] = sum_k |S[n][k/G] * x[m][k]|           (normaliser of the parity check)
 * Either output pointer may be NULL. */
void oracle_gemv(const uint16_t *x, const uint32_t *W, const uint16_t *S,
                 int64_t M, int64_t K, int64_t N, int64_t G,
                 double *y, double *nrm)
{
    const int64_t wpr = (K + 31) / 32;
    const int64_t spr = K / G;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; ++n) {
        const uint32_t *row = W + n * wpr;
        const uint16_t *srow = S + n * spr;
        for (int64_t m = 0; m < M; ++m) {
            const uint16_t *xr = x + m * K;
            double acc = 0.0, a = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double s = oracle_half_to_double(srow[k / G]);
                double xv = oracle_half_to_double(xr[k]);
                acc += s * weight_sign(row, k) * xv;
                a += fabs(s * xv);
            }
            if (y) y[m * N + n] = acc;
            if (nrm) nrm[m * N + n] = a;
        }
    }
}

/* Ternary weight of (n, k) from its 2-bit slot ("Bonsai 27B", section on the ternary weight
 * format: t in {-1, 0, +1}, w = s_g * t, one fp16 scale per group of 128; the same page's
 * deployment section: current kernels keep each ternary value in a 2-bit slot).  Reading:
 * slot k % 16 of word k / 16, LSB first; within the slot, the low bit says nonzero and the
 * high bit says negative (00 -> 0, 01 -> +1, 11 -> -1; 10, never written, reads as 0). */
static inline double ternary_value(const uint32_t *row, int64_t k)
{
    const uint32_t code = (row[k / 16] >> (2 * (k % 16))) & 3u;
    if (!(code & 1u)) return 0.0;
    return (code & 2u) ? -1.0 : 1.0;
}

/* y[m][n]   = sum_k S[n][k/G] * t(n,k) * x[m][k]   (ascending k, fp64)
 * nrm[m][n] = sum_k |S[n][k/G] * t(n,k) * x[m][k]| (parity normaliser: the terms the product
 * actually adds).  T: uint32 [N][ceil(K/16)].  Either output pointer may be NULL. */
void oracle_gemv_t2(const uint16_t *x, const uint32_t *T, const uint16_t *S,
                    int64_t M, int64_t K, int64_t N, int64_t G, double *y, double *nrm)
{
    const int64_t wpr = (K + 15) / 16;
    const int64_t spr = K / G;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; ++n) {
        const uint32_t *row = T + n * wpr;
        const uint16_t *srow = S + n * spr;
        for (int64_t m = 0; m < M; ++m) {
            const uint16_t *xr = x + m * K;
            double acc = 0.0, a = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double term = oracle_half_to_double(srow[k / G]) * ternary_value(row, k) *
                              oracle_half_to_double(xr[k]);
                acc += term;
                a += fabs(term);
            }
            if (y) y[m * N + n] = acc;
            if (nrm) nrm[m * N + n] = a;
        }
    }
}

/* +-1 activations and weights, both packed (bit 1 = +1):
 * y[m][n] = sum_k a(m,k) * w(n,k), exact in int64. */
void oracle_pm1(const uint32_t *A, const uint32_t *W,
                int64_t M, int64_t K, int64_t N, int64_t *y)
{
    const int64_t wpr = (K + 31) / 32;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; ++n) {
        const uint32_t *row = W + n * wpr;
        for (int64_t m = 0; m < M; ++m) {
            const uint32_t *arow = A + m * wpr;
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t a = ((arow[k / 32] >> (k % 32)) & 1u) ? 1 : -1;
                int64_t w = ((row[k / 32] >> (k % 32)) & 1u) ? 1 : -1;
                acc += a * w;
            }
            y[m * N + n] = acc;
        }
    }
}

/* XOR row patch, in place: every word of each listed row is complemented
 * (flipping all K signs of output row r).  Entries outside [0, N) are skipped
 * and counted; the count is returned.  Applying the same list twice restores W. */
int64_t oracle_xor_patch(uint32_t *W, int64_t K, int64_t N,
                         const int32_t *rows, int64_t nrows)
{
    const int64_t wpr = (K + 31) / 32;
    int64_t bad = 0;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows[i];
        if (r < 0 || r >= N) { ++bad; continue; }
        for (int64_t j = 0; j < wpr; ++j)
            W[r * wpr + j] ^= 0xFFFFFFFFu;
    }
    return bad;
}

/* Bit-granular XOR patch over a set of matrices ("LocalLLaMA ... XOR patch 'Bankai'",
 * sections on the experiments -- random flips of single bits of the MLP weights -- and on
 * why XOR patches need true binary codes): entry i = (matrix id, row, k) flips the sign bit
 * of weight k of that row.  Entries are applied one after another, so a bit listed an even
 * number of times is unchanged and the same list applied twice restores every matrix.
 * Entries with id outside [0, nmat), row outside [0, N_id), k outside [0, K_id), or a K_id
 * that is not a positive multiple of 128 are skipped and counted; the count is returned.
 * Wtab holds host pointers to the matrices ([N_id][K_id/32] uint32 each). */
int64_t oracle_xor_bits(uint32_t *const *Wtab, const int64_t *Ktab, const int64_t *Ntab,
                        int64_t nmat, const int32_t *entries, int64_t nentries)
{
    int64_t bad = 0;
    for (int64_t i = 0; i < nentries; ++i) {
        const int64_t id = entries[3 * i], r = entries[3 * i + 1], k = entries[3 * i + 2];
        if (id < 0 || id >= nmat) { ++bad; continue; }
        const int64_t K = Ktab[id], N = Ntab[id];
        if (K <= 0 || K % 128 != 0 || r < 0 || r >= N || k < 0 || k >= K) { ++bad; continue; }
        Wtab[id][r * (K / 32) + k / 32] ^= (uint32_t)1u << (k % 32);
    }
    return bad;
}

/* Scale-ranked rows (the Bankai page's scale-factor targeting, experiments section): the
 * score of row n is the sum over its groups of |S[n][g]|, taken exactly as an integer in
 * units of 2^-24, the spacing of the smallest fp16 subnormal:
 *   |s| = frac * 2^-24 for exponent 0, (1024 + frac) * 2^(expo - 25) otherwise,
 * so |s| * 2^24 = frac or (1024 + frac) << (expo - 1) (for exponent 31, inf/NaN, the same
 * formula is used; it exceeds every finite value).  order receives the rows by score,
 * largest first, equal scores by ascending row. */
static const int64_t *rank_score;
static int rank_cmp(const void *a, const void *b)
{
    const int32_t i = *(const int32_t *)a, j = *(const int32_t *)b;
    if (rank_score[i] != rank_score[j]) return rank_score[i] > rank_score[j] ? -1 : 1;
    return i < j ? -1 : (i > j);
}

void oracle_rank_rows(const uint16_t *S, int64_t N, int64_t groups, int64_t *score, int32_t *order)
{
    for (int64_t n = 0; n < N; ++n) {
        int64_t acc = 0;
        for (int64_t g = 0; g < groups; ++g) {
            const uint16_t h = S[n * groups + g];
            const int64_t expo = (h >> 10) & 0x1f, frac = h & 0x3ff;
            acc += expo == 0 ? frac : ((1024 + frac) << (expo - 1));
        }
        score[n] = acc;
        order[n] = (int32_t)n;
    }
    rank_score = score;
    qsort(order, (size_t)N, sizeof(int32_t), rank_cmp);
}

int oracle_max_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }
