// gemv_chain.hip -- a chain of dependent batch-1 decode stages in one persistent launch.
//
// A decode step is a sequence of stages (q/k/v, o, gate/up, down per layer, then lm_head);
// every stage is one or more sign-weight GEMVs that read the same activation vector, and a
// stage may start only when the previous one has finished.  At batch 1 the pages observe that
// datacenter GPUs are bound by launch and synchronisation latency rather than weight
// bandwidth ["Bonsai 27B" page, section "Low-bit kernels for hybrid attention", the H100
// batch-1 remark].  This kernel removes the per-stage launches: one workgroup per CU stays
// resident for the whole chain, weights of the next stage are already streaming while a
// stage waits for its predecessor, and the inter-stage dependency is a device-scope
// release/acquire handshake through per-workgroup flags in a caller-owned workspace.
//
// The per-stage product is the block-scaled MFMA decode of gemv_mx.hip (fp4 sign expansion,
// fp8 activation limbs), restricted to K % 256 == 0 (an even number of scale groups).
//
// Work split: every stage is cut into units of `rt` row tiles (16 rows each) of one matrix, and
// the 256 workgroups take units round-robin.  A workgroup's 4 waves split K into 1024-wide pairs
// (wave w takes pairs w, w+4, ...).  A prefetch slot holds SP (row tile, pair) blocks per wave, so
// a stage with one pair per wave packs SP row tiles into a unit and keeps as many bytes in flight
// as a stage with SP pairs per wave.
//
// Workspace (caller-owned device memory, laid out by bin1_chain_prepare):
//   ChainHeader | done flags [nstages][kChainWgs] int32 | ChainStage table [nstages]
// Flags and the run generation only grow, so the kernel can be replayed (from a HIP graph)
// without clearing anything: run number g waits for flags >= g + 1.
#include "common.hpp"
#include "kernels.hpp"
#include "mx_common.hpp"

#include <type_traits>

namespace bin1 {

namespace {

using namespace mx;

constexpr long kSpinLimit = 1L << 21;           // polls before a wait gives up (seconds)
constexpr int kSc1 = 16;                         // buffer cache policy: device-scope coherent
constexpr int kStageWords = sizeof(ChainStage) / 4;
static_assert(sizeof(ChainStage) % 8 == 0, "stage descriptors are copied as whole words");

__device__ __forceinline__ int ld_relaxed(const int *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Values read from the LDS copy of the stage table are wave-uniform; moving them to SGPRs keeps
// buffer resources and loop bounds scalar.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <class T>
__device__ __forceinline__ T *unip(T *p)
{
    const unsigned long long v = reinterpret_cast<unsigned long long>(p);
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
    return reinterpret_cast<T *>(((unsigned long long)hi << 32) | lo);
}

__device__ __forceinline__ int units_of(int nunits, int me)
{
    return me < nunits ? (nunits - 1 - me) / kChainWgs + 1 : 0;
}

template <int SP>
struct CSlot {
    u4v w[SP][2];       // block b: this lane's 32 bytes (two groups) of its row and pair
    uint32_t s[SP];     // block b: the two groups' fp16 scales
};

// Where global unit `gu` (wave-uniform) of stage `st` lies: its matrix and first row.  The
// matrix index is found first, then only that matrix's fields are read (few live scalar
// registers).
struct UnitAt {
    int mi, N, row0;
};

__device__ __forceinline__ UnitAt unit_at(const ChainStage &st, int gu)
{
    const int count = uni(st.count), rows = 16 * uni(st.rt);
    int mi = 0, start = 0;
#pragma unroll
    for (int i = 0; i < kMaxMats - 1; ++i) {
        const int e = uni(st.unit_end[i]);
        if (i + 1 < count && gu >= e) { mi = i + 1; start = e; }
    }
    return UnitAt{mi, uni(st.N[mi]), (gu - start) * rows};
}

// The same for a per-lane unit index (the merge, where lanes cover different units): every
// matrix's fields are read as uniform values and the lane selects among them.
__device__ __forceinline__ void unit_at_lane(const ChainStage &st, int gu, uint16_t *&y, int &N, int &row0)
{
    const int count = uni(st.count), rows = 16 * uni(st.rt);
    y = unip(st.y[0]);
    N = uni(st.N[0]);
    int start = 0;
#pragma unroll
    for (int i = 1; i < kMaxMats; ++i) {
        const int e = uni(st.unit_end[i - 1]), Ni = uni(st.N[i]);
        uint16_t *yi = unip(st.y[i]);
        if (i < count && gu >= e) { y = yi; N = Ni; start = e; }
    }
    row0 = (gu - start) * rows;
}

template <int I, int MAX, class F>
__device__ __forceinline__ void dispatch_npw(int npw, F &&f)
{
    if constexpr (I <= MAX) {
        if (npw == I) f(std::integral_constant<int, I>{});
        else dispatch_npw<I + 1, MAX>(npw, f);
    }
}

// Stage handoff.  Every HIP fence or release/acquire at device scope writes back or invalidates
// a whole XCD L2 on this GPU, and 256 workgroups doing so per stage costs far more than the
// stage itself.  The handoff therefore uses only device-scope-coherent accesses (cache policy
// SC1), which the hardware keeps coherent across XCDs without cache maintenance:
//   producer: outputs stored with SC1; s_waitcnt until every store is acknowledged; barrier;
//             one SC1 flag store per workgroup;
//   consumer: wave 0 polls the 256 flags with SC1 loads; barrier; x is loaded with SC1 when
//             some stage of the chain writes it.
// The only data passed between stages are those outputs, so no other cache traffic needs
// ordering: weights, the stage table and an x that no stage writes are read-only for the whole
// launch and may come from L2.
template <int SP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemv_chain_kernel(ChainHeader *hdr, int *done, const ChainStage *table, int nst, long spin_limit)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int me = blockIdx.x;
    const int target = ld_relaxed(&hdr->gen) + 1;
    const bool withhold = me == 0 && ld_relaxed(&hdr->withhold) != 0;

    // LDS: stage table | per-wave limb blocks [4][2*SP segments][4 words] x kBlk | per-wave
    // exponent dwords [4][2*SP][16] | merge table [tiles][16 rows][4 waves] fp32.
    const int tbytes = (nst * (int)sizeof(ChainStage) + 15) & ~15;
    ChainStage *lt = reinterpret_cast<ChainStage *>(lds);
    uint8_t *lwave = lds + tbytes + wave * (2 * SP * 4 * kBlk);
    uint32_t *scw = reinterpret_cast<uint32_t *>(lds + tbytes + 4 * (2 * SP * 4 * kBlk)) + wave * (2 * SP * 16);
    float *red = reinterpret_cast<float *>(lds + tbytes + 4 * (2 * SP * 4 * kBlk) + 4 * (2 * SP * 16) * 4);
    {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(table);
        uint32_t *dst = reinterpret_cast<uint32_t *>(lds);
        for (int i = tid; i < nst * kStageWords; i += 256) dst[i] = src[i];
    }
    for (int i = lane; i < 2 * SP * 4; i += 64)        // zero bytes of every block (never overwritten)
        *reinterpret_cast<u4v *>(lwave + i * kBlk + kZero) = u4v{0, 0, 0, 0};
    __syncthreads();

    int lo, hi;
    a_offsets(lane, lo, hi);
    const int m = lane & 15;

    // Prefetch unit = (stage, index among this workgroup's units of that stage).  issue_at looks
    // the unit up (LDS reads only); issue starts its loads.
    struct IssueAt {
        const uint32_t *W;
        const uint16_t *S;
        int N, K, rt, row0;
        bool live;
    };
    auto issue_at = [&](int s, int u) {
        const bool live = s < nst;
        const ChainStage &st = lt[live ? s : 0];
        const UnitAt a = unit_at(st, me + u * kChainWgs);
        return IssueAt{unip(st.W[a.mi]), unip(st.S[a.mi]), a.N, uni(st.K), uni(st.rt), a.row0, live};
    };
    auto issue = [&](const IssueAt &d, CSlot<SP> &sl) {
        const int wpr = d.K >> 5, spr = d.K >> 7;
        const int npw = chain_pairs_per_wave(d.K);
        const __amdgpu_buffer_rsrc_t rW = rsrc(d.W, (unsigned)d.N * (unsigned)wpr * 4u);
        const __amdgpu_buffer_rsrc_t rS = rsrc(d.S, (unsigned)d.N * (unsigned)spr * 2u);
#pragma unroll
        for (int b = 0; b < SP; ++b) {
            const int t = b / npw, p = b - t * npw;    // row tile, pair of block b
            const int row = d.row0 + 16 * t + n;
            const int gam = 8 * (wave + 4 * p) + 2 * g;
            const bool ok = d.live && t < d.rt && row < d.N && gam < spr;   // K % 256 == 0: gam+1 valid
            // mul24 row products (rows < 2^24) keep the wait counts exact
            const unsigned ow = (mul24((unsigned)row, (unsigned)wpr) + 4u * gam) * 4u;
            const unsigned os = (mul24((unsigned)row, (unsigned)spr) + gam) * 2u;
            sl.w[b][0] = __builtin_amdgcn_raw_buffer_load_b128(rW, ok ? ow : kOob, 0, kNT);
            sl.w[b][1] = __builtin_amdgcn_raw_buffer_load_b128(rW, ok ? ow + 16u : kOob, 0, kNT);
            sl.s[b] = __builtin_amdgcn_raw_buffer_load_b32(rS, ok ? os : kOob, 0, 0);
        }
    };
    // next unit after (s, u), skipping stages where this workgroup has none
    auto advance = [&](int &s, int &u) {
        ++u;
        while (s < nst && u >= units_of(uni(lt[s].nunits), me)) { ++s; u = 0; }
    };

    CSlot<SP> ring[2];
    int is = 0, iu = -1;                               // issue cursor: last unit issued
    advance(is, iu);
    issue(issue_at(is, iu), ring[0]);
    advance(is, iu);
    issue(issue_at(is, iu), ring[1]);
    int cur = 0;                                       // ring slot of the next unit to compute

    for (int s = 0; s < nst; ++s) {
        const ChainStage &st = lt[s];
        const int K = uni(st.K), rt = uni(st.rt), nunits = uni(st.nunits);
        const uint16_t *xp = unip(st.x);
        const bool xsc1 = uni(st.x_written) != 0;
        const int nmine = units_of(nunits, me);
        const int npair = (K + 1023) >> 10, npw = chain_pairs_per_wave(K);
        // ---- wait for the previous stage: every workgroup's flag >= target.  Wave 0 polls (one
        // poller per workgroup keeps the 256 flags' lines from becoming a hot spot) with two polls
        // in flight, issued half a round trip apart and each re-issued as soon as it returns.
        if (s > 0) {
            if (wave == 0) {
                const int *f = done + (size_t)(s - 1) * kChainWgs + lane;
                auto seen = [&](int f0, int f1, int f2, int f3) {
                    return __all(f0 >= target && f1 >= target && f2 >= target && f3 >= target);
                };
                long spins = 0;
                int a0 = ld_relaxed(f), a1 = ld_relaxed(f + 64), a2 = ld_relaxed(f + 128), a3 = ld_relaxed(f + 192);
                __builtin_amdgcn_s_sleep(16);
                int b0 = ld_relaxed(f), b1 = ld_relaxed(f + 64), b2 = ld_relaxed(f + 128), b3 = ld_relaxed(f + 192);
                int be = ld_relaxed(&hdr->error);
                for (;;) {
                    if (seen(a0, a1, a2, a3)) break;
                    a0 = ld_relaxed(f); a1 = ld_relaxed(f + 64); a2 = ld_relaxed(f + 128); a3 = ld_relaxed(f + 192);
                    if (seen(b0, b1, b2, b3)) break;
                    // give up after the spin limit, or at once if another workgroup already did
                    if (++spins > spin_limit || be) {
                        if (lane == 0) __hip_atomic_store(&hdr->error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    b0 = ld_relaxed(f); b1 = ld_relaxed(f + 64); b2 = ld_relaxed(f + 128); b3 = ld_relaxed(f + 192);
                    be = ld_relaxed(&hdr->error);
                }
            }
            __syncthreads();
        }
        if (nmine == 0) {                              // nothing of this stage here: just signal
            if (tid == 0 && !(withhold && s == 0))
                __hip_atomic_store(done + (size_t)s * kChainWgs + me, target, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            continue;
        }
        const __amdgpu_buffer_rsrc_t rx = rsrc(xp, (unsigned)K * 2u);
        // Everything below is specialised on NPW = pairs per wave of this stage: x conversion and
        // the A operands cover exactly those pairs, and a unit holds RT = SP / NPW row tiles.
        dispatch_npw<1, SP>(npw, [&](auto npw_c) {
            constexpr int NPW = decltype(npw_c)::value, RT = SP / NPW;
            // ---- this wave's pairs of x -> limbs (wave-local LDS) -> A registers
            int8v A[NPW][2][4];
            int scA[NPW][2];
#pragma unroll
            for (int q = 0; q < NPW; ++q) {
                const int pr = wave + 4 * q;
                const unsigned off = (unsigned)(1024 * pr + 16 * lane) * 2u;
                u4v p0, p1;
                if (xsc1) {                            // x is written inside the chain
                    p0 = __builtin_amdgcn_raw_buffer_load_b128(rx, pr < npair ? off : kOob, 0, kSc1);
                    p1 = __builtin_amdgcn_raw_buffer_load_b128(rx, pr < npair ? off + 16u : kOob, 0, kSc1);
                } else {                               // read-only for the whole launch: L2 may serve it
                    p0 = __builtin_amdgcn_raw_buffer_load_b128(rx, pr < npair ? off : kOob, 0, 0);
                    p1 = __builtin_amdgcn_raw_buffer_load_b128(rx, pr < npair ? off + 16u : kOob, 0, 0);
                }
                float mx = absmax16(p0, p1);
                mx = fmaxf(mx, __shfl_xor(mx, 1, kWave));
                const int beta = lane >> 1, h = lane & 1;  // 32-block within the pair
                const int gamma = beta >> 2, t = beta & 3; // group within the pair (0..7), word
                const int lseg = 2 * q + (gamma & 1), G4 = gamma >> 1;
                convert16(p0, p1, mx, lwave + (lseg * 4 + t) * kBlk, G4, h,
                          reinterpret_cast<uint8_t *>(scw) + (lseg * 16 + 4 * G4) * 4 + t);
            }
#pragma unroll
            for (int q = 0; q < NPW; ++q)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) A[q][h][t] = load_a(lwave + ((2 * q + h) * 4 + t) * kBlk, lo, hi);
                    scA[q][h] = (int)scw[(2 * q + h) * 16 + m];
                }
            // ---- this workgroup's units of stage s.  Slots alternate; the two loops differ only
            // in which slot comes first, so within a loop the wait for a slot's loads is a fixed
            // count and the other slot's loads stay in flight.
            float *rb = red;
            auto one = [&](CSlot<SP> &sl) {
                advance(is, iu);                       // (is, iu) = last unit issued; look up the
                const IssueAt nx = issue_at(is, iu);   // next one before the products run
                // All blocks' MFMA chains advance together, word by word, so consecutive MFMAs
                // are independent (one accumulator per chain) and the matrix pipe stays full.
                // Branch-free: a block past the end of K has zero activations and zero scales
                // (out-of-range loads), so it adds exactly 0, and straight-line code lets the
                // compiler keep the other slot's loads in flight.
                constexpr int NB = RT * NPW;
                float4v c[NB][2];
#pragma unroll
                for (int b = 0; b < NB; ++b) c[b][0] = c[b][1] = float4v{0.f, 0.f, 0.f, 0.f};
                auto word = [&](auto T_c) {
                    constexpr int T = decltype(T_c)::value;
#pragma unroll
                    for (int b = 0; b < NB; ++b)
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int p = b % NPW;
                            c[b][h] = mma<T>(A[p][h][T], sl.w[b][h][T], scA[p][h], c[b][h]);
                        }
                };
                word(std::integral_constant<int, 0>{});
                word(std::integral_constant<int, 1>{});
                word(std::integral_constant<int, 2>{});
                word(std::integral_constant<int, 3>{});
                float acc[RT];
#pragma unroll
                for (int t = 0; t < RT; ++t) acc[t] = 0.f;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const uint32_t sv = sl.s[b];
                    const float s0 = h2f((uint16_t)(sv & 0xFFFFu)), s1 = h2f((uint16_t)(sv >> 16));
                    // B held -w, so a group's partial is -(c0+c1+c2+c3)
                    acc[b / NPW] = fmaf(-s0, (c[b][0][0] + c[b][0][1]) + (c[b][0][2] + c[b][0][3]), acc[b / NPW]);
                    acc[b / NPW] = fmaf(-s1, (c[b][1][0] + c[b][1][1]) + (c[b][1][2] + c[b][1][3]), acc[b / NPW]);
                }
                issue(nx, sl);                         // refill this slot with that unit
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    const float v = sum_groups(acc[t]);
                    if (lane < 16) rb[(16 * t + lane) * 4 + wave] = v;
                }
                rb += 64 * RT;
            };
            int left = nmine;
            if (cur == 0) {
                for (;;) {
                    one(ring[0]);
                    if (--left == 0) { cur = 1; break; }
                    one(ring[1]);
                    if (--left == 0) break;
                }
            } else {
                for (;;) {
                    one(ring[1]);
                    if (--left == 0) { cur = 0; break; }
                    one(ring[0]);
                    if (--left == 0) break;
                }
            }
        });
        __syncthreads();
        // ---- merge the waves' K-slices, store y (device-scope coherent), publish
        const int urows = 16 * rt;
        for (int e = tid; e < nmine * urows; e += 256) {
            const int u = e / urows, j = e - u * urows;
            uint16_t *y;
            int N, row0;
            unit_at_lane(st, me + u * kChainWgs, y, N, row0);
            const int row = row0 + j;
            const float4v p4 = *reinterpret_cast<const float4v *>(red + e * 4);
            if (row < N)
                __hip_atomic_store(y + row, f2h_rne((p4[0] + p4[1]) + (p4[2] + p4[3])), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0): every output store acknowledged
        __syncthreads();
        if (tid == 0 && !(withhold && s == 0))
            __hip_atomic_store(done + (size_t)s * kChainWgs + me, target, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0) {
        const int prev = __hip_atomic_fetch_add(&hdr->exit_count, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == target * kChainWgs - 1)
            __hip_atomic_store(&hdr->gen, target, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
}

size_t lds_need(int sp, int nst, int max_tiles)
{
    return (size_t)((nst * (int)sizeof(ChainStage) + 15) & ~15) + (size_t)4 * (2 * sp * 4 * kBlk) +
           (size_t)4 * (2 * sp * 16) * 4 + (size_t)max_tiles * 64 * 4;
}

constexpr size_t kMaxLds = 160 * 1024;

template <int SP>
hipError_t launch_chain_t(ChainHeader *hdr, int *done, const ChainStage *table, int nst, int max_tiles,
                          long spin_limit, hipStream_t st)
{
    const size_t shm = lds_need(SP, nst, max_tiles);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&gemv_chain_kernel<SP>), hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)kMaxLds);
    if (attr != hipSuccess) return attr;
    if (shm > kMaxLds) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemv_chain_kernel<SP>), dim3(kChainWgs), dim3(256), shm, st, hdr, done, table, nst,
                       spin_limit);
    return hipGetLastError();
}

}  // namespace

size_t chain_lds_bytes(int spmax, int nstages, int max_tiles)
{
    const size_t b = lds_need(spmax, nstages, max_tiles);
    return b <= kMaxLds ? b : 0;
}

hipError_t launch_gemv_chain(ChainHeader *hdr, int *done, const ChainStage *table, int nst, int spmax,
                             int max_tiles, long spin_limit, hipStream_t st)
{
    if (spin_limit <= 0) spin_limit = kSpinLimit;
    switch (spmax) {
    case 1: return launch_chain_t<1>(hdr, done, table, nst, max_tiles, spin_limit, st);
    case 2: return launch_chain_t<2>(hdr, done, table, nst, max_tiles, spin_limit, st);
    case 3: return launch_chain_t<3>(hdr, done, table, nst, max_tiles, spin_limit, st);
    case 4: return launch_chain_t<4>(hdr, done, table, nst, max_tiles, spin_limit, st);
    case 5: return launch_chain_t<5>(hdr, done, table, nst, max_tiles, spin_limit, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace bin1
