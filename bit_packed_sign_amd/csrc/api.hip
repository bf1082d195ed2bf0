// api.hip -- the C ABI of libbin1 (declared in include/bin1.h): argument validation,
// dispatch to the kernels, status codes and the thread-local error text.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "bin1.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok()
{
    g_last_error.clear();
    return BIN1_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

// The pointer must be device memory (or managed memory) visible on the current device.
// Allocation ranges that passed are remembered per thread (a few of them, most recent first):
// a later pointer inside one of them, on the same device, is accepted without a new runtime query.
struct Validated {
    uintptr_t base, end;
    int device;
};
thread_local Validated g_valid[16];
thread_local int g_nvalid = 0;

int check_device(const void *p, const char *name)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(BIN1_ERR_DEVICE, "%s: no current HIP device", name);
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    for (int i = 0; i < g_nvalid; ++i)
        if (g_valid[i].device == dev && a >= g_valid[i].base && a < g_valid[i].end) {
            if (i > 0) std::swap(g_valid[i], g_valid[0]);
            return BIN1_OK;
        }
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(BIN1_ERR_DEVICE, "%s: not a HIP allocation (%s)", name, hipGetErrorString(e));
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
        return fail(BIN1_ERR_DEVICE, "%s: not device memory (memory type %d)", name, (int)attr.type);
    if (attr.device != dev)
        return fail(BIN1_ERR_DEVICE, "%s: allocated on device %d, current device is %d", name,
                    attr.device, dev);
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void *>(p)) == hipSuccess && size > 0) {
        const int slot = g_nvalid < 16 ? g_nvalid++ : 15;
        for (int i = slot; i > 0; --i) g_valid[i] = g_valid[i - 1];
        g_valid[0] = Validated{reinterpret_cast<uintptr_t>(base), reinterpret_cast<uintptr_t>(base) + size, dev};
    } else {
        (void)hipGetLastError();
    }
    return BIN1_OK;
}

int launched(hipError_t e, const char *what)
{
    if (e != hipSuccess) return fail(BIN1_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Shared validation of the (x, Wbits, scales, y, M, K, N) products: host-side checks first.
// bits: bits per weight of W (1: signs, 2: ternary slots)
// Returns kEmpty (> 0) for a product with no outputs (M == 0 or N == 0): nothing to compute,
// and its pointers are not used.
constexpr int kEmpty = 1;

int check_product_host(const void *x, const void *W, const void *S, const void *y, int M, int K, int N,
                       int bits = 1)
{
    if (M < 0 || N < 0 || K < 128 || K % 128 != 0)
        return fail(BIN1_ERR_SHAPE, "need M>=0, N>=0, K>=128, K%%128==0 (got M=%d K=%d N=%d)", M, K, N);
    if (M == 0 || N == 0) return kEmpty;
    if (!x || !W || !S || !y) return fail(BIN1_ERR_NULL, "x, Wbits, scales and y must be non-NULL");
    if (!aligned16(x) || !aligned16(W) || !aligned16(S) || !aligned16(y))
        return fail(BIN1_ERR_ALIGN, "x, Wbits, scales and y must be 16-byte aligned");
    const size_t xb = (size_t)M * K * 2, wb = (size_t)N * (K / 8) * bits, sb = (size_t)N * (K / 128) * 2,
                 yb = (size_t)M * N * 2;
    // the kernels address rows with 24-bit products and buffers with 32-bit offsets
    if (N >= (1 << 24) - 64 || xb >= (1ull << 31) || wb >= (1ull << 31) || yb >= (1ull << 31))
        return fail(BIN1_ERR_SHAPE, "need N < 2^24 - 64 and x, Wbits, y each under 2 GiB (got M=%d K=%d N=%d)", M,
                    K, N);
    if (overlap(y, yb, x, xb) || overlap(y, yb, W, wb) || overlap(y, yb, S, sb))
        return fail(BIN1_ERR_ALIAS, "y overlaps an input");
    return BIN1_OK;
}

int check_product_device(const void *x, const void *W, const void *S, const void *y)
{
    int st;
    if ((st = check_device(x, "x")) || (st = check_device(W, "Wbits")) ||
        (st = check_device(S, "scales")) || (st = check_device(y, "y")))
        return st;
    return BIN1_OK;
}

int check_product(const void *x, const void *W, const void *S, const void *y, int M, int K, int N, int bits = 1)
{
    int st = check_product_host(x, W, S, y, M, K, N, bits);
    return st ? st : check_product_device(x, W, S, y);
}

}  // namespace

namespace bin1 {

int set_error(int status, const char *what) { return fail(status, "%s", what); }

// bin1_gemv with a scratch area for the split-K path.  caller_ws: the scratch is the caller's
// (validated like the other pointers); otherwise it is the library's own static array.
int gemv_scratch(const char *fn, const void *x, const uint32_t *Wbits, const void *scales, void *y, int M, int K,
                 int N, void *ws, size_t ws_bytes, bool caller_ws, void *stream)
{
    int st = check_product_host(x, Wbits, scales, y, M, K, N);
    if (st) return st == kEmpty ? ok() : st;
    const size_t need = smallm_split_bytes(M, K, N);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (need == 0) {
        if ((st = check_product_device(x, Wbits, scales, y))) return st;
        return launched(launch_gemv(static_cast<const uint16_t *>(x), Wbits, static_cast<const uint16_t *>(scales),
                                    static_cast<uint16_t *>(y), M, K, N, s),
                        fn);
    }
    if (!ws) return fail(BIN1_ERR_NULL, "%s: this shape needs %zu bytes of workspace", fn, need);
    if (ws_bytes < need)
        return fail(BIN1_ERR_SHAPE, "%s: workspace of %zu bytes, this shape needs %zu", fn, ws_bytes, need);
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(BIN1_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
    if (caller_ws) {
        const size_t xb = (size_t)M * K * 2, wb = (size_t)N * (K / 8), sb = (size_t)N * (K / 128) * 2,
                     yb = (size_t)M * N * 2;
        if (overlap(ws, need, x, xb) || overlap(ws, need, Wbits, wb) || overlap(ws, need, scales, sb) ||
            overlap(ws, need, y, yb))
            return fail(BIN1_ERR_ALIAS, "%s: the workspace overlaps an input or the output", fn);
    }
    if ((st = check_product_device(x, Wbits, scales, y)) || (caller_ws && (st = check_device(ws, "workspace"))))
        return st;
    MxSet set{};
    set.W[0] = Wbits;
    set.S[0] = static_cast<const uint16_t *>(scales);
    set.y[0] = static_cast<uint16_t *>(y);
    set.N[0] = N;
    set.count = 1;
    return launched(launch_gemv_smallm(static_cast<const uint16_t *>(x), set, M, K, s, nullptr, static_cast<float *>(ws)),
                    fn);
}

}  // namespace bin1

extern "C" {

int bin1_abi_version(void) { return BIN1_ABI_VERSION; }

const char *bin1_last_error(void) { return g_last_error.c_str(); }

size_t bin1_chain_workspace_bytes(int nstages)
{
    if (nstages < 1) return 0;
    const size_t flags = (size_t)nstages * bin1::kChainWgs * sizeof(int);
    const size_t table = (size_t)nstages * sizeof(bin1::ChainStage);
    return sizeof(bin1::ChainHeader) + ((flags + 255) & ~(size_t)255) + table;
}

int bin1_chain_prepare(const bin1_stage *stages, int nstages, void *workspace, size_t workspace_bytes,
                       bin1_chain_plan *plan)
{
    if (!stages || !workspace || !plan) return fail(BIN1_ERR_NULL, "stages, workspace and plan must be non-NULL");
    if (nstages < 1) return fail(BIN1_ERR_SHAPE, "need nstages >= 1");
    const size_t need = bin1_chain_workspace_bytes(nstages);
    if (workspace_bytes < need)
        return fail(BIN1_ERR_SHAPE, "workspace too small: %zu bytes, need %zu", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(BIN1_ERR_ALIGN, "workspace must be 256-byte aligned");
    int st;
    if ((st = check_device(workspace, "workspace"))) return st;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return fail(BIN1_ERR_DEVICE, "cannot query the device");
    if (cus < bin1::kChainWgs)
        return fail(BIN1_ERR_DEVICE, "the chain needs %d compute units, the device has %d", bin1::kChainWgs, cus);
    int spmax = 1;
    for (int s = 0; s < nstages; ++s) {
        const bin1_stage &g = stages[s];
        if (g.count < 1 || g.count > bin1::kMaxMats)
            return fail(BIN1_ERR_SHAPE, "stage %d: count must be 1..%d", s, bin1::kMaxMats);
        if (g.K < 256 || g.K % 256 != 0 || g.K > 20 * 1024)
            return fail(BIN1_ERR_SHAPE, "stage %d: K must be a multiple of 256 in [256, 20480] (got %d)", s, g.K);
        const int sp = ((g.K >> 10) + 3) / 4;
        if (sp > spmax) spmax = sp;
        for (int i = 0; i < g.count; ++i) {
            if (g.N[i] < 1) return fail(BIN1_ERR_SHAPE, "stage %d: every product needs N >= 1", s);
            if ((st = check_product_host(g.x, g.Wbits[i], g.scales[i], g.y[i], 1, g.K, g.N[i]))) return st;
            if ((st = check_product_device(g.x, g.Wbits[i], g.scales[i], g.y[i]))) return st;
        }
    }
    // outputs must not overwrite any weight or scale of the chain, nor another output of their stage
    for (int s = 0; s < nstages; ++s)
        for (int i = 0; i < stages[s].count; ++i) {
            const void *y = stages[s].y[i];
            const size_t yb = (size_t)stages[s].N[i] * 2;
            for (int t = 0; t < nstages; ++t)
                for (int j = 0; j < stages[t].count; ++j) {
                    const bin1_stage &u = stages[t];
                    if (overlap(y, yb, u.Wbits[j], (size_t)u.N[j] * (u.K / 8)) ||
                        overlap(y, yb, u.scales[j], (size_t)u.N[j] * (u.K / 128) * 2) ||
                        (t == s && j != i && overlap(y, yb, u.y[j], (size_t)u.N[j] * 2)))
                        return fail(BIN1_ERR_ALIAS, "stage %d output %d overlaps stage %d matrix %d", s, i, t, j);
                }
        }
    std::vector<bin1::ChainStage> table(nstages);
    int max_tiles = 0;
    for (int s = 0; s < nstages; ++s) {
        const bin1_stage &g = stages[s];
        bin1::ChainStage &c = table[s];
        memset(&c, 0, sizeof c);
        c.x = static_cast<const uint16_t *>(g.x);
        c.K = g.K;
        c.count = g.count;
        c.rt = bin1::chain_unit_tiles(spmax, g.K);
        const int urows = 16 * c.rt;
        int units = 0;
        for (int i = 0; i < g.count; ++i) {
            c.W[i] = g.Wbits[i];
            c.S[i] = static_cast<const uint16_t *>(g.scales[i]);
            c.y[i] = static_cast<uint16_t *>(g.y[i]);
            c.N[i] = g.N[i];
            units += (g.N[i] + urows - 1) / urows;
            c.unit_end[i] = units;
        }
        c.nunits = units;
        for (int t = 0; t < nstages && !c.x_written; ++t)
            for (int j = 0; j < stages[t].count; ++j)
                if (overlap(g.x, (size_t)g.K * 2, stages[t].y[j], (size_t)stages[t].N[j] * 2)) c.x_written = 1;
        const int tiles = (units + bin1::kChainWgs - 1) / bin1::kChainWgs * c.rt;   // workgroup 0 has the most
        if (tiles > max_tiles) max_tiles = tiles;
    }
    if (bin1::chain_lds_bytes(spmax, nstages, max_tiles) == 0)
        return fail(BIN1_ERR_SHAPE, "the chain does not fit in on-chip memory (%d stages, %d row tiles per "
                    "workgroup in its largest stage)", nstages, max_tiles);
    bin1::ChainHeader hdr;
    memset(&hdr, 0, sizeof hdr);
    hdr.nstages = nstages;
    hdr.spmax = spmax;
    hdr.max_tiles = max_tiles;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    const size_t flags = (size_t)nstages * bin1::kChainWgs * sizeof(int);
    const size_t toff = sizeof(bin1::ChainHeader) + ((flags + 255) & ~(size_t)255);
    hipError_t e = hipMemcpy(ws, &hdr, sizeof hdr, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemset(ws + sizeof(bin1::ChainHeader), 0, flags);
    if (e == hipSuccess) e = hipMemcpy(ws + toff, table.data(), table.size() * sizeof(bin1::ChainStage),
                                       hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(BIN1_ERR_LAUNCH, "bin1_chain_prepare: %s", hipGetErrorString(e));
    plan->workspace = workspace;
    plan->nstages = nstages;
    plan->spmax = spmax;
    plan->max_tiles = max_tiles;
    plan->spin_limit = 0;
    return ok();
}

int bin1_gemv_chain(const bin1_chain_plan *plan, void *stream)
{
    if (!plan || !plan->workspace) return fail(BIN1_ERR_NULL, "plan and its workspace must be non-NULL");
    if (plan->nstages < 1 || plan->spmax < 1 || plan->spmax > 5)
        return fail(BIN1_ERR_SHAPE, "plan was not prepared");
    if (plan->spin_limit < 0) return fail(BIN1_ERR_SHAPE, "spin_limit must be >= 0");
    uint8_t *ws = static_cast<uint8_t *>(plan->workspace);
    const size_t flags = (size_t)plan->nstages * bin1::kChainWgs * sizeof(int);
    const size_t toff = sizeof(bin1::ChainHeader) + ((flags + 255) & ~(size_t)255);
    return launched(bin1::launch_gemv_chain(reinterpret_cast<bin1::ChainHeader *>(ws),
                                            reinterpret_cast<int *>(ws + sizeof(bin1::ChainHeader)),
                                            reinterpret_cast<const bin1::ChainStage *>(ws + toff),
                                            plan->nstages, plan->spmax, plan->max_tiles, plan->spin_limit,
                                            static_cast<hipStream_t>(stream)),
                    "bin1_gemv_chain");
}

int bin1_chain_status(const bin1_chain_plan *plan, int *runs, int *error)
{
    if (!plan || !plan->workspace || !runs || !error) return fail(BIN1_ERR_NULL, "NULL argument");
    bin1::ChainHeader hdr;
    hipError_t e = hipMemcpy(&hdr, plan->workspace, sizeof hdr, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(BIN1_ERR_LAUNCH, "bin1_chain_status: %s", hipGetErrorString(e));
    *runs = hdr.gen;
    *error = hdr.error;
    return ok();
}

const char *bin1_status_string(int status)
{
    switch (status) {
    case BIN1_OK: return "BIN1_OK";
    case BIN1_ERR_NULL: return "BIN1_ERR_NULL: a required pointer is NULL";
    case BIN1_ERR_SHAPE: return "BIN1_ERR_SHAPE: a size is out of range";
    case BIN1_ERR_ALIGN: return "BIN1_ERR_ALIGN: a data pointer is not 16-byte aligned";
    case BIN1_ERR_ALIAS: return "BIN1_ERR_ALIAS: the output overlaps an input";
    case BIN1_ERR_DEVICE: return "BIN1_ERR_DEVICE: a pointer is not device memory of the current device";
    case BIN1_ERR_LAUNCH: return "BIN1_ERR_LAUNCH: the HIP runtime refused the launch";
    default: return "unknown bin1 status";
    }
}

int bin1_gemv(const void *x, const uint32_t *Wbits, const void *scales, void *y, int M, int K,
              int N, void *stream)
{
    int st = check_product(x, Wbits, scales, y, M, K, N);
    if (st) return st == kEmpty ? ok() : st;
    return launched(bin1::launch_gemv(static_cast<const uint16_t *>(x), Wbits,
                                      static_cast<const uint16_t *>(scales),
                                      static_cast<uint16_t *>(y), M, K, N,
                                      static_cast<hipStream_t>(stream)),
                    "bin1_gemv");
}

}  // extern "C"

namespace {

// Launches of the same-input products of 1..4 matrices (validated, back-to-back ones already merged);
// with `desc`, describes them instead (the variant query).  t2: ternary weights in 2-bit slots.
hipError_t route_group(bool t2, const void *x, int count, const uint32_t *const *Wbits, const void *const *scales,
                       void *const *y, const int *N, int M, int K, hipStream_t st, std::string *desc)
{
    if (M == 1 && K <= bin1::mx_max_k()) {
        bin1::MxSet set{};
        int tiles = 0;
        for (int i = 0; i < count; ++i) {
            set.W[i] = Wbits[i];
            set.S[i] = static_cast<const uint16_t *>(scales[i]);
            set.y[i] = static_cast<uint16_t *>(y[i]);
            set.N[i] = N[i];
            tiles += (N[i] + 15) / 16;
            set.tile_end[i] = tiles;
        }
        set.count = count;
        return t2 ? bin1::launch_gemv_mx_t2(static_cast<const uint16_t *>(x), set, K, st, desc)
                  : bin1::launch_gemv_mx(static_cast<const uint16_t *>(x), set, K, st, desc);
    }
    if (t2) {                                             // other batch sizes: the prefill kernel
        for (int i = 0; i < count; ++i) {
            hipError_t e = bin1::launch_prefill_t2(static_cast<const uint16_t *>(x), Wbits[i],
                                                   static_cast<const uint16_t *>(scales[i]),
                                                   static_cast<uint16_t *>(y[i]), M, K, N[i], st, desc);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    if (M >= 2 && M <= 16) {                              // small batch: one launch as well
        bin1::MxSet set{};
        for (int i = 0; i < count; ++i) {
            set.W[i] = Wbits[i];
            set.S[i] = static_cast<const uint16_t *>(scales[i]);
            set.y[i] = static_cast<uint16_t *>(y[i]);
            set.N[i] = N[i];
        }
        set.count = count;
        return bin1::launch_gemv_smallm(static_cast<const uint16_t *>(x), set, M, K, st, desc);
    }
    for (int i = 0; i < count; ++i) {
        hipError_t e = bin1::launch_gemv(static_cast<const uint16_t *>(x), Wbits[i],
                                         static_cast<const uint16_t *>(scales[i]),
                                         static_cast<uint16_t *>(y[i]), M, K, N[i], st, desc);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Ternary product of one matrix: M == 1 on the block-scaled decode kernel, other M on the prefill kernel.
hipError_t route_t2(const void *x, const uint32_t *Tbits, const void *scales, void *y, int M, int K, int N,
                    hipStream_t s, std::string *desc)
{
    if (M == 1 && K <= bin1::mx_max_k()) {
        bin1::MxSet set{};
        set.W[0] = Tbits;
        set.S[0] = static_cast<const uint16_t *>(scales);
        set.y[0] = static_cast<uint16_t *>(y);
        set.N[0] = N;
        set.count = 1;
        return bin1::launch_gemv_mx_t2(static_cast<const uint16_t *>(x), set, K, s, desc);
    }
    return bin1::launch_prefill_t2(static_cast<const uint16_t *>(x), Tbits, static_cast<const uint16_t *>(scales),
                                   static_cast<uint16_t *>(y), M, K, N, s, desc);
}

// Same-input products of 1..4 matrices; t2: ternary weights in 2-bit slots.
int gemv_group_impl(const char *fn, bool t2, const void *x, int count, const uint32_t *const *Wbits,
                    const void *const *scales, void *const *y, const int *N, int M, int K, void *stream)
{
    const int bits = t2 ? 2 : 1;
    if (count < 1 || count > bin1::kMaxMats)
        return fail(BIN1_ERR_SHAPE, "count must be 1..%d (got %d)", bin1::kMaxMats, count);
    if (!Wbits || !scales || !y || !N) return fail(BIN1_ERR_NULL, "pointer arrays must be non-NULL");
    // products with no outputs (M == 0 or N[i] == 0) are dropped; the rest go ahead
    int live[bin1::kMaxMats], nlive = 0;
    for (int i = 0; i < count; ++i) {
        const int st = check_product_host(x, Wbits[i], scales[i], y[i], M, K, N[i], bits);
        if (st < 0) return st;
        if (st != kEmpty) live[nlive++] = i;
    }
    if (nlive == 0) return ok();
    // every output against every other product's inputs and output, on the caller's list (before
    // any merge below, so that an output touching a neighbour's weights is still caught)
    for (int a = 0; a < nlive; ++a)
        for (int b = 0; b < nlive; ++b) {
            const int i = live[a], j = live[b];
            if (i == j) continue;
            const size_t yb = (size_t)M * N[i] * 2;
            if (overlap(y[i], yb, y[j], (size_t)M * N[j] * 2) ||
                overlap(y[i], yb, Wbits[j], (size_t)N[j] * (K / 8) * bits) ||
                overlap(y[i], yb, scales[j], (size_t)N[j] * (K / 128) * 2))
                return fail(BIN1_ERR_ALIAS, "y[%d] overlaps an input or output of matrix %d", i, j);
        }
    const uint32_t *Wk[bin1::kMaxMats];
    const void *Sk[bin1::kMaxMats];
    void *yk[bin1::kMaxMats];
    int Nk[bin1::kMaxMats], kept = 0;
    for (int a = 0; a < nlive; ++a) {
        const int i = live[a];
        // At M == 1, a matrix stored right after the previous kept one (its weights, scales and
        // outputs each start where the previous one's end, as in a fused q/k/v layout) extends
        // that one: rows are independent, so the taller matrix gives the same products.
        if (M == 1 && kept > 0) {
            const int p = kept - 1;
            const size_t n = (size_t)Nk[p], nn = n + (size_t)N[i];
            const bool adjacent = Wbits[i] == Wk[p] + n * (size_t)(K / 32) * bits &&
                                  scales[i] == static_cast<const char *>(Sk[p]) + n * (size_t)(K / 128) * 2 &&
                                  y[i] == static_cast<char *>(yk[p]) + n * 2;
            if (adjacent && nn < (1u << 24) - 64 && nn * (size_t)(K / 8) * bits < (1ull << 31)) {
                Nk[p] = (int)nn;
                continue;
            }
        }
        Wk[kept] = Wbits[i];
        Sk[kept] = scales[i];
        yk[kept] = y[i];
        Nk[kept++] = N[i];
    }
    int st;
    if ((st = check_device(x, "x"))) return st;
    for (int i = 0; i < kept; ++i)
        if ((st = check_device(Wk[i], "Wbits")) || (st = check_device(Sk[i], "scales")) ||
            (st = check_device(yk[i], "y")))
            return st;
    return launched(route_group(t2, x, kept, Wk, Sk, yk, Nk, M, K, static_cast<hipStream_t>(stream), nullptr), fn);
}

}  // namespace

extern "C" {

int bin1_gemv_group(const void *x, int count, const uint32_t *const *Wbits, const void *const *scales,
                    void *const *y, const int *N, int M, int K, void *stream)
{
    return gemv_group_impl("bin1_gemv_group", false, x, count, Wbits, scales, y, N, M, K, stream);
}

int bin1_gemv_group_t2(const void *x, int count, const uint32_t *const *Tbits, const void *const *scales,
                       void *const *y, const int *N, int M, int K, void *stream)
{
    return gemv_group_impl("bin1_gemv_group_t2", true, x, count, Tbits, scales, y, N, M, K, stream);
}

int bin1_gemm_prefill(const void *x, const uint32_t *Wbits, const void *scales, void *y, int M,
                      int K, int N, void *stream)
{
    int st = check_product(x, Wbits, scales, y, M, K, N);
    if (st) return st == kEmpty ? ok() : st;
    return launched(bin1::launch_prefill(static_cast<const uint16_t *>(x), Wbits,
                                         static_cast<const uint16_t *>(scales),
                                         static_cast<uint16_t *>(y), M, K, N,
                                         static_cast<hipStream_t>(stream)),
                    "bin1_gemm_prefill");
}

int bin1_gemv_pm1(const uint32_t *Abits, const uint32_t *Wbits, int32_t *y, int M, int K, int N,
                  void *stream)
{
    if (M < 0 || N < 0 || K < 128 || K % 128 != 0)
        return fail(BIN1_ERR_SHAPE, "need M>=0, N>=0, K>=128, K%%128==0 (got M=%d K=%d N=%d)", M, K, N);
    if (M == 0 || N == 0) return ok();                 // no outputs
    if (!Abits || !Wbits || !y) return fail(BIN1_ERR_NULL, "Abits, Wbits and y must be non-NULL");
    if (!aligned16(Abits) || !aligned16(Wbits) || !aligned16(y))
        return fail(BIN1_ERR_ALIGN, "Abits, Wbits and y must be 16-byte aligned");
    const size_t ab = (size_t)M * (K / 8), wb = (size_t)N * (K / 8), yb = (size_t)M * N * 4;
    if (overlap(y, yb, Abits, ab) || overlap(y, yb, Wbits, wb))
        return fail(BIN1_ERR_ALIAS, "y overlaps an input");
    int st;
    if ((st = check_device(Abits, "Abits")) || (st = check_device(Wbits, "Wbits")) ||
        (st = check_device(y, "y")))
        return st;
    return launched(bin1::launch_pm1(Abits, Wbits, y, M, K, N, static_cast<hipStream_t>(stream)),
                    "bin1_gemv_pm1");
}

int bin1_xor_patch_apply(uint32_t *Wbits, const int32_t *rowlist, int nrows, int K, int N,
                         int32_t *bad_rows, void *stream)
{
    if (nrows < 0 || N < 1 || K < 128 || K % 128 != 0)
        return fail(BIN1_ERR_SHAPE, "need nrows>=0, N>=1, K>=128, K%%128==0 (got nrows=%d K=%d N=%d)",
                    nrows, K, N);
    if (nrows == 0) return ok();
    if (!Wbits || !rowlist) return fail(BIN1_ERR_NULL, "Wbits and rowlist must be non-NULL");
    if (!aligned16(Wbits)) return fail(BIN1_ERR_ALIGN, "Wbits must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(rowlist) & 3u || reinterpret_cast<uintptr_t>(bad_rows) & 3u)
        return fail(BIN1_ERR_ALIGN, "rowlist and bad_rows must be 4-byte aligned");
    const size_t wb = (size_t)N * (K / 8);
    if (overlap(Wbits, wb, rowlist, (size_t)nrows * 4) || (bad_rows && overlap(Wbits, wb, bad_rows, 4)))
        return fail(BIN1_ERR_ALIAS, "Wbits overlaps rowlist or bad_rows");
    int st;
    if ((st = check_device(Wbits, "Wbits")) || (st = check_device(rowlist, "rowlist")) ||
        (bad_rows && (st = check_device(bad_rows, "bad_rows"))))
        return st;
    return launched(bin1::launch_xor_patch(Wbits, rowlist, nrows, K, N, bad_rows,
                                           static_cast<hipStream_t>(stream)),
                    "bin1_xor_patch_apply");
}

int bin1_xor_patch_apply_multi(uint32_t *const *Wtab, const int32_t *Ktab, const int32_t *Ntab,
                               int nmat, const int32_t *entries, int nentries, int32_t *bad_rows,
                               void *stream)
{
    if (nentries < 0 || nmat < 1)
        return fail(BIN1_ERR_SHAPE, "need nentries>=0 and nmat>=1 (got %d, %d)", nentries, nmat);
    if (nentries == 0) return ok();
    if (!Wtab || !Ktab || !Ntab || !entries)
        return fail(BIN1_ERR_NULL, "Wtab, Ktab, Ntab and entries must be non-NULL");
    if (reinterpret_cast<uintptr_t>(Wtab) & 7u || reinterpret_cast<uintptr_t>(Ktab) & 3u ||
        reinterpret_cast<uintptr_t>(Ntab) & 3u || reinterpret_cast<uintptr_t>(entries) & 3u ||
        reinterpret_cast<uintptr_t>(bad_rows) & 3u)
        return fail(BIN1_ERR_ALIGN, "tables must be naturally aligned");
    int st;
    if ((st = check_device(Wtab, "Wtab")) || (st = check_device(Ktab, "Ktab")) ||
        (st = check_device(Ntab, "Ntab")) || (st = check_device(entries, "entries")) ||
        (bad_rows && (st = check_device(bad_rows, "bad_rows"))))
        return st;
    return launched(bin1::launch_xor_patch_multi(Wtab, Ktab, Ntab, nmat, entries, nentries, bad_rows,
                                                 static_cast<hipStream_t>(stream)),
                    "bin1_xor_patch_apply_multi");
}

int bin1_xor_bits_apply(uint32_t *const *Wtab, const int32_t *Ktab, const int32_t *Ntab, int nmat,
                        const int32_t *entries, int nentries, int32_t *bad, void *stream)
{
    if (nentries < 0 || nmat < 1)
        return fail(BIN1_ERR_SHAPE, "need nentries>=0 and nmat>=1 (got %d, %d)", nentries, nmat);
    if (nentries == 0) return ok();
    if (!Wtab || !Ktab || !Ntab || !entries)
        return fail(BIN1_ERR_NULL, "Wtab, Ktab, Ntab and entries must be non-NULL");
    if (reinterpret_cast<uintptr_t>(Wtab) & 7u || reinterpret_cast<uintptr_t>(Ktab) & 3u ||
        reinterpret_cast<uintptr_t>(Ntab) & 3u || reinterpret_cast<uintptr_t>(entries) & 3u ||
        reinterpret_cast<uintptr_t>(bad) & 3u)
        return fail(BIN1_ERR_ALIGN, "tables must be naturally aligned");
    int st;
    if ((st = check_device(Wtab, "Wtab")) || (st = check_device(Ktab, "Ktab")) ||
        (st = check_device(Ntab, "Ntab")) || (st = check_device(entries, "entries")) ||
        (bad && (st = check_device(bad, "bad"))))
        return st;
    return launched(bin1::launch_xor_bits(Wtab, Ktab, Ntab, nmat, entries, nentries, bad,
                                          static_cast<hipStream_t>(stream)),
                    "bin1_xor_bits_apply");
}

int bin1_rank_rows_by_scale(const void *scales, int N, int K, int64_t *score, int32_t *order, void *stream)
{
    if (N < 0 || N > (1 << 20) || K < 128 || K % 128 != 0)
        return fail(BIN1_ERR_SHAPE, "need 0 <= N <= 2^20, K >= 128, K %% 128 == 0 (got N=%d K=%d)", N, K);
    if (N == 0) return ok();                           // no rows to rank
    if (!scales || !score || !order) return fail(BIN1_ERR_NULL, "scales, score and order must be non-NULL");
    if (!aligned16(scales) || reinterpret_cast<uintptr_t>(score) & 7u || reinterpret_cast<uintptr_t>(order) & 3u)
        return fail(BIN1_ERR_ALIGN, "scales must be 16-byte aligned, score 8-byte, order 4-byte");
    const size_t sb = (size_t)N * (K / 128) * 2, cb = (size_t)N * 8, ob = (size_t)N * 4;
    if (overlap(score, cb, scales, sb) || overlap(order, ob, scales, sb) || overlap(order, ob, score, cb))
        return fail(BIN1_ERR_ALIAS, "scales, score and order must not overlap");
    int st;
    if ((st = check_device(scales, "scales")) || (st = check_device(score, "score")) ||
        (st = check_device(order, "order")))
        return st;
    return launched(bin1::launch_rank_rows(static_cast<const uint16_t *>(scales), N, K, score, order,
                                           static_cast<hipStream_t>(stream)),
                    "bin1_rank_rows_by_scale");
}

int bin1_gemv_t2(const void *x, const uint32_t *Tbits, const void *scales, void *y, int M, int K, int N,
                 void *stream)
{
    int st = check_product(x, Tbits, scales, y, M, K, N, 2);
    if (st) return st == kEmpty ? ok() : st;
    return launched(route_t2(x, Tbits, scales, y, M, K, N, static_cast<hipStream_t>(stream), nullptr),
                    "bin1_gemv_t2");
}

int bin1_gemm_prefill_t2(const void *x, const uint32_t *Tbits, const void *scales, void *y, int M, int K, int N,
                         void *stream)
{
    int st = check_product(x, Tbits, scales, y, M, K, N, 2);
    if (st) return st == kEmpty ? ok() : st;
    return launched(bin1::launch_prefill_t2(static_cast<const uint16_t *>(x), Tbits,
                                            static_cast<const uint16_t *>(scales), static_cast<uint16_t *>(y),
                                            M, K, N, static_cast<hipStream_t>(stream)),
                    "bin1_gemm_prefill_t2");
}

int bin1_stream_read(const void *buf, size_t bytes, uint32_t *sink, int grid, int unroll, void *stream)
{
    if (bytes == 0 || bytes % 16 != 0 || grid < 1 || grid > 65536 || (unroll != 4 && unroll != 8 && unroll != 16))
        return fail(BIN1_ERR_SHAPE, "need bytes a positive multiple of 16, 1 <= grid <= 65536, unroll 4, 8 or 16 "
                    "(got %zu, %d, %d)", bytes, grid, unroll);
    if (!buf || !sink) return fail(BIN1_ERR_NULL, "buf and sink must be non-NULL");
    if (!aligned16(buf) || reinterpret_cast<uintptr_t>(sink) & 3u)
        return fail(BIN1_ERR_ALIGN, "buf must be 16-byte aligned and sink 4-byte aligned");
    if (overlap(sink, (size_t)grid * 16, buf, bytes)) return fail(BIN1_ERR_ALIAS, "sink overlaps buf");
    int st;
    if ((st = check_device(buf, "buf")) || (st = check_device(sink, "sink"))) return st;
    return launched(bin1::launch_stream_read(buf, bytes, sink, grid, unroll, static_cast<hipStream_t>(stream)),
                    "bin1_stream_read");
}

int bin1_mfma_rate(const void *operands, float *sink, int grid, int waves, int iters, void *stream)
{
    if (grid < 1 || grid > 65536 || (waves != 4 && waves != 8) || iters < 1 || iters > 1000000)
        return fail(BIN1_ERR_SHAPE, "need 1 <= grid <= 65536, waves 4 or 8, 1 <= iters <= 1000000 (got %d, %d, %d)",
                    grid, waves, iters);
    if (!operands || !sink) return fail(BIN1_ERR_NULL, "operands and sink must be non-NULL");
    if (!aligned16(operands) || reinterpret_cast<uintptr_t>(sink) & 3u)
        return fail(BIN1_ERR_ALIGN, "operands must be 16-byte aligned and sink 4-byte aligned");
    if (overlap(sink, (size_t)grid * waves * 4, operands, 2048)) return fail(BIN1_ERR_ALIAS, "sink overlaps operands");
    int st;
    if ((st = check_device(operands, "operands")) || (st = check_device(sink, "sink"))) return st;
    return launched(bin1::launch_mfma_rate(operands, sink, grid, waves, iters, static_cast<hipStream_t>(stream)),
                    "bin1_mfma_rate");
}

int bin1_kernel_variant(int op, int M, int K, int count, const int *N, char *name, int len)
{
    if (!N || !name) return fail(BIN1_ERR_NULL, "N and name must be non-NULL");
    if (len < 1) return fail(BIN1_ERR_SHAPE, "len must be >= 1");
    name[0] = 0;
    if (op < 0 || op > 4 || count < 1 || count > bin1::kMaxMats || (op >= 2 && count != 1))
        return fail(BIN1_ERR_SHAPE, "need op 0..4 and count 1..%d (1 for ops 2..4)", bin1::kMaxMats);
    if (M < 1 || K < 128 || K % 128 != 0)
        return fail(BIN1_ERR_SHAPE, "need M >= 1, K >= 128, K %% 128 == 0 (got M=%d K=%d)", M, K);
    for (int i = 0; i < count; ++i)
        if (N[i] < 1 || N[i] >= (1 << 24) - 64) return fail(BIN1_ERR_SHAPE, "N[%d] out of range (%d)", i, N[i]);
    // Stand-in addresses, never dereferenced (nothing is launched): distinct, aligned, and not back
    // to back, as the caller's matrices after any merge.
    const uint32_t *W[bin1::kMaxMats];
    const void *S[bin1::kMaxMats];
    void *Y[bin1::kMaxMats];
    for (int i = 0; i < bin1::kMaxMats; ++i) {
        W[i] = reinterpret_cast<const uint32_t *>((uintptr_t)(0x100000000ull * (1 + i)));
        S[i] = reinterpret_cast<const void *>((uintptr_t)(0x100000000ull * (5 + i)));
        Y[i] = reinterpret_cast<void *>((uintptr_t)(0x100000000ull * (9 + i)));
    }
    const void *X = reinterpret_cast<const void *>((uintptr_t)0x1000000000ull);
    std::string desc;
    hipError_t e = hipSuccess;
    switch (op) {
    case 0:
        e = count == 1 ? bin1::launch_gemv(static_cast<const uint16_t *>(X), W[0], static_cast<const uint16_t *>(S[0]),
                                           static_cast<uint16_t *>(Y[0]), M, K, N[0], nullptr, &desc)
                       : route_group(false, X, count, W, S, Y, N, M, K, nullptr, &desc);
        break;
    case 1:
        e = count == 1 ? route_t2(X, W[0], S[0], Y[0], M, K, N[0], nullptr, &desc)
                       : route_group(true, X, count, W, S, Y, N, M, K, nullptr, &desc);
        break;
    case 2:
        e = bin1::launch_prefill(static_cast<const uint16_t *>(X), W[0], static_cast<const uint16_t *>(S[0]),
                                 static_cast<uint16_t *>(Y[0]), M, K, N[0], nullptr, &desc);
        break;
    case 3:
        e = bin1::launch_prefill_t2(static_cast<const uint16_t *>(X), W[0], static_cast<const uint16_t *>(S[0]),
                                    static_cast<uint16_t *>(Y[0]), M, K, N[0], nullptr, &desc);
        break;
    default:                                          // bin1_gemv_ws with a large enough workspace
        if (bin1::smallm_split_bytes(M, K, N[0]) == 0) {
            e = bin1::launch_gemv(static_cast<const uint16_t *>(X), W[0], static_cast<const uint16_t *>(S[0]),
                                  static_cast<uint16_t *>(Y[0]), M, K, N[0], nullptr, &desc);
        } else {
            bin1::MxSet set{};
            set.W[0] = W[0];
            set.S[0] = static_cast<const uint16_t *>(S[0]);
            set.y[0] = static_cast<uint16_t *>(Y[0]);
            set.N[0] = N[0];
            set.count = 1;
            e = bin1::launch_gemv_smallm(static_cast<const uint16_t *>(X), set, M, K, nullptr, &desc,
                                         reinterpret_cast<float *>((uintptr_t)0x2000000000ull));
        }
        break;
    }
    if (e != hipSuccess) return fail(BIN1_ERR_LAUNCH, "bin1_kernel_variant: %s", hipGetErrorString(e));
    if ((int)desc.size() >= len) return fail(BIN1_ERR_SHAPE, "name buffer too small: need %zu bytes", desc.size() + 1);
    memcpy(name, desc.c_str(), desc.size() + 1);
    return ok();
}

size_t bin1_gemv_workspace_bytes(int M, int K, int N)
{
    if (M < 1 || N < 1 || K < 128 || K % 128 != 0) return 0;
    return bin1::smallm_split_bytes(M, K, N);
}

int bin1_gemv_ws(const void *x, const uint32_t *Wbits, const void *scales, void *y, int M, int K, int N,
                 void *workspace, size_t workspace_bytes, void *stream)
{
    return bin1::gemv_scratch("bin1_gemv_ws", x, Wbits, scales, y, M, K, N, workspace, workspace_bytes, true, stream);
}

}  // extern "C"
