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
// Workspace (caller-owned device memory, laid out by bin1_chain_prepare):
//   ChainHeader | done flags [nstages][kChainWgs] int32 | ChainStage table [nstages]
// Flags and the run generation only grow, so the kernel can be replayed (from a HIP graph)
// without clearing anything: run number g waits for flags >= g + 1.
#include "common.hpp"
#include "kernels.hpp"
#include "mx_common.hpp"

namespace bin1 {

namespace {

using namespace mx;

constexpr long kSpinLimit = 1L << 21;           // polls before a wait gives up (seconds)
constexpr int kSc1 = 16;                         // buffer cache policy: device-scope coherent

// The stage table never changes while the kernel runs: reading it through the constant address
// space gives scalar loads, so descriptors and buffer resources stay in SGPRs and table reads
// never wait behind the weight loads in flight.
typedef const __attribute__((address_space(4))) ChainStage CStage;

__device__ __forceinline__ int ld_relaxed(const int *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int SP, int R>
struct CSlot {
    u4v w[R][SP][2];
    uint32_t s[R][SP];
};

__device__ __forceinline__ void chain_locate(CStage &st, int tile, int R, int &mi, int &row0)
{
    mi = 0;
#pragma unroll
    for (int i = 0; i < kMaxMats - 1; ++i)
        if (i + 1 < st.count && tile >= st.tile_end[i]) mi = i + 1;
    row0 = (tile - (mi ? st.tile_end[mi - 1] : 0)) * 16 * R;
}

__device__ __forceinline__ int tiles_of(int ntiles, int me)
{
    return me < ntiles ? (ntiles - 1 - me) / kChainWgs + 1 : 0;
}

// Stage handoff.  Every HIP fence or release/acquire at device scope writes back or invalidates
// a whole XCD L2 on this GPU, and 256 workgroups doing so per stage costs far more than the
// stage itself.  The handoff therefore uses only device-scope-coherent accesses (cache policy
// SC1), which the hardware keeps coherent across XCDs without cache maintenance:
//   producer: outputs stored with SC1; s_waitcnt until every store is acknowledged; barrier;
//             one SC1 flag store per workgroup;
//   consumer: SC1 polls of the 256 flags; barrier; activations loaded with SC1.
// The only data passed between stages are those outputs, so no other cache traffic needs
// ordering (weights and the stage table are read-only).
template <int SP, int R>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemv_chain_kernel(ChainHeader *hdr, int *done, const ChainStage *table_, int nst, long spin_limit)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    CStage *table = (CStage *)table_;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int me = blockIdx.x;
    const int target = ld_relaxed(&hdr->gen) + 1;
    const bool withhold = me == 0 && ld_relaxed(&hdr->withhold) != 0;

    // LDS: per-wave limb blocks [4 waves][2*SP segments][4 words] x kBlk, per-wave exponent
    // dwords [4][2*SP][16], then the merge table [tiles][16R rows][4 waves] fp32.
    uint8_t *lwave = lds + wave * (2 * SP * 4 * kBlk);
    uint32_t *scw = reinterpret_cast<uint32_t *>(lds + 4 * (2 * SP * 4 * kBlk)) + wave * (2 * SP * 16);
    float *red = reinterpret_cast<float *>(lds + 4 * (2 * SP * 4 * kBlk) + 4 * (2 * SP * 16) * 4);
    // zero bytes of every block (never overwritten)
    for (int i = lane; i < 2 * SP * 4; i += 64)
        *reinterpret_cast<u4v *>(lwave + i * kBlk + kZero) = u4v{0, 0, 0, 0};

    int lo, hi;
    a_offsets(lane, lo, hi);
    const int m = lane & 15;

    // Prefetch unit = (stage, tile index among this workgroup's tiles of that stage).
    auto issue = [&](int s, int it, CSlot<SP, R> &sl) {
        const bool live = s < nst;
        CStage &st = table[live ? s : 0];
        const bool tl = live && it < tiles_of(st.ntiles, me);
        int mi, row0;
        chain_locate(st, tl ? me + it * kChainWgs : 0, R, mi, row0);
        const int K = st.K, wpr = K >> 5, spr = K >> 7, N = st.N[mi];
        const __amdgpu_buffer_rsrc_t rW = rsrc(st.W[mi], (unsigned)N * (unsigned)wpr * 4u);
        const __amdgpu_buffer_rsrc_t rS = rsrc(st.S[mi], (unsigned)N * (unsigned)spr * 2u);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = row0 + 16 * r + n;
            const bool rok = tl && row < N;
#pragma unroll
            for (int q = 0; q < SP; ++q) {
                const int gam = 8 * (wave + 4 * q) + 2 * g;
                const bool ok = rok && gam < spr;        // K % 256 == 0: gam+1 valid too
                const unsigned ow = ((unsigned)row * wpr + 4u * gam) * 4u;
                const unsigned os = ((unsigned)row * spr + gam) * 2u;
                sl.w[r][q][0] = __builtin_amdgcn_raw_buffer_load_b128(rW, ok ? ow : kOob, 0, kNT);
                sl.w[r][q][1] = __builtin_amdgcn_raw_buffer_load_b128(rW, ok ? ow + 16u : kOob, 0, kNT);
                sl.s[r][q] = __builtin_amdgcn_raw_buffer_load_b32(rS, ok ? os : kOob, 0, 0);
            }
        }
    };
    // next unit after (s, it): the following tile of this workgroup, skipping empty stages
    auto advance = [&](int &s, int &it) {
        ++it;
        while (s < nst && it >= tiles_of(table[s].ntiles, me)) { ++s; it = 0; }
    };

    CSlot<SP, R> ring[2];
    int is = 0, ii = -1;                               // issue cursor: last unit issued
    advance(is, ii);
    issue(is, ii, ring[0]);
    advance(is, ii);
    issue(is, ii, ring[1]);
    int cur = 0;                                       // ring slot of the next unit to compute

    for (int s = 0; s < nst; ++s) {
        CStage &st = table[s];
        const int nmine = tiles_of(st.ntiles, me);
        // ---- wait for the previous stage: every workgroup's flag >= target
        if (s > 0) {
            if (wave == 0) {
                long spins = 0;
                const int *f = done + (size_t)(s - 1) * kChainWgs + lane;
                for (;;) {
                    const int f0 = ld_relaxed(f), f1 = ld_relaxed(f + 64);
                    const int f2 = ld_relaxed(f + 128), f3 = ld_relaxed(f + 192);
                    const int err = ld_relaxed(&hdr->error);
                    if (__all(f0 >= target && f1 >= target && f2 >= target && f3 >= target)) break;
                    // give up after the spin limit, or at once if another workgroup already did
                    if (++spins > spin_limit || err) {
                        if (lane == 0) __hip_atomic_store(&hdr->error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
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
        // ---- this wave's K-slice of x -> limbs (wave-local LDS) -> A registers
        const int K = st.K, npair = (K + 1023) >> 10;   // last pair may hold only 2..6 groups
        const __amdgpu_buffer_rsrc_t rx = rsrc(st.x, (unsigned)K * 2u);
#pragma unroll
        for (int q = 0; q < SP; ++q) {
            const int pr = wave + 4 * q;
            const unsigned off = (unsigned)(1024 * pr + 16 * lane) * 2u;
            const u4v p0 = __builtin_amdgcn_raw_buffer_load_b128(rx, pr < npair ? off : kOob, 0, kSc1);
            const u4v p1 = __builtin_amdgcn_raw_buffer_load_b128(rx, pr < npair ? off + 16u : kOob, 0, kSc1);
            float mx = absmax16(p0, p1);
            mx = fmaxf(mx, __shfl_xor(mx, 1, kWave));
            const int beta = lane >> 1, h = lane & 1;  // 32-block within the pair
            const int gamma = beta >> 2, t = beta & 3; // group within the pair (0..7), word
            const int lseg = 2 * q + (gamma & 1), G4 = gamma >> 1;
            convert16(p0, p1, mx, lwave + (lseg * 4 + t) * kBlk, G4, h,
                      reinterpret_cast<uint8_t *>(scw) + (lseg * 16 + 4 * G4) * 4 + t);
        }
        int8v A[SP][2][4];
        int scA[SP][2];
#pragma unroll
        for (int q = 0; q < SP; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int t = 0; t < 4; ++t) A[q][h][t] = load_a(lwave + ((2 * q + h) * 4 + t) * kBlk, lo, hi);
                scA[q][h] = (int)scw[(2 * q + h) * 16 + m];
            }
        // ---- this workgroup's tiles of stage s.  Slots alternate; the two loops differ only
        // in which slot comes first, so within a loop the wait for a slot's loads is a fixed
        // count and the other slot's loads stay in flight.
        float *rb = red;
        auto body = [&](CSlot<SP, R> &sl) {
            float acc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
            for (int q = 0; q < SP; ++q) {
                const int pr = wave + 4 * q;
                if (pr < npair) {
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const uint32_t sv = sl.s[r][q];
                        const float s0 = h2f((uint16_t)(sv & 0xFFFFu)), s1 = h2f((uint16_t)(sv >> 16));
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const u4v w = sl.w[r][q][h];
                            float4v c = {0.f, 0.f, 0.f, 0.f};
                            c = mma<0>(A[q][h][0], w.x, scA[q][h], c);
                            c = mma<1>(A[q][h][1], w.y, scA[q][h], c);
                            c = mma<2>(A[q][h][2], w.z, scA[q][h], c);
                            c = mma<3>(A[q][h][3], w.w, scA[q][h], c);
                            acc[r] = fmaf(-(h ? s1 : s0), (c[0] + c[1]) + (c[2] + c[3]), acc[r]);
                        }
                    }
                }
            }
            advance(is, ii);                           // (is, ii) = last unit issued
            issue(is, ii, sl);                         // refill this slot with the one after it
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float v = sum_groups(acc[r]);
                if (lane < 16) rb[(16 * r + lane) * 4 + wave] = v;
            }
            rb += 64 * R;
        };
        int left = nmine;
        if (cur == 0) {
            for (;;) {
                body(ring[0]);
                if (--left == 0) { cur = 1; break; }
                body(ring[1]);
                if (--left == 0) break;
            }
        } else {
            for (;;) {
                body(ring[1]);
                if (--left == 0) { cur = 0; break; }
                body(ring[0]);
                if (--left == 0) break;
            }
        }
        __syncthreads();
        // ---- merge the waves' K-slices, store y (device-scope coherent), publish
        for (int e = tid; e < nmine * 16 * R; e += 256) {
            const int it = e / (16 * R), j = e - it * (16 * R);
            int mi, row0;
            chain_locate(st, me + it * kChainWgs, R, mi, row0);
            const int row = row0 + j;
            const float4v p4 = *reinterpret_cast<const float4v *>(red + e * 4);
            // select among the (scalar) descriptors rather than index them per lane
            int Nm = st.N[0];
            uint16_t *ym = st.y[0];
#pragma unroll
            for (int i = 1; i < kMaxMats; ++i)
                if (mi == i) { Nm = st.N[i]; ym = st.y[i]; }
            if (row < Nm)
                __hip_atomic_store(ym + row, f2h_rne((p4[0] + p4[1]) + (p4[2] + p4[3])), __ATOMIC_RELAXED,
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

template <int SP, int R>
size_t chain_lds(int max_tiles)
{
    return (size_t)4 * (2 * SP * 4 * kBlk) + 4 * (2 * SP * 16) * 4 + (size_t)max_tiles * 64 * R * 4;
}

template <int SP, int R>
hipError_t launch_chain_t(ChainHeader *hdr, int *done, const ChainStage *table, int nst, int max_tiles,
                          long spin_limit, hipStream_t st)
{
    const size_t shm = chain_lds<SP, R>(max_tiles);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&gemv_chain_kernel<SP, R>), hipFuncAttributeMaxDynamicSharedMemorySize,
        160 * 1024);
    if (attr != hipSuccess) return attr;
    if (shm > 160 * 1024) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemv_chain_kernel<SP, R>), dim3(kChainWgs), dim3(256), shm, st, hdr, done, table, nst,
                       spin_limit);
    return hipGetLastError();
}

}  // namespace

int chain_rows_per_tile(int spmax) { return spmax <= 2 ? 32 : 16; }

hipError_t launch_gemv_chain(ChainHeader *hdr, int *done, const ChainStage *table, int nst, int spmax,
                             int max_tiles, long spin_limit, hipStream_t st)
{
    if (spin_limit <= 0) spin_limit = kSpinLimit;
    switch (spmax) {
    case 1: return launch_chain_t<1, 2>(hdr, done, table, nst, max_tiles, spin_limit, st);
    case 2: return launch_chain_t<2, 2>(hdr, done, table, nst, max_tiles, spin_limit, st);
    case 3: return launch_chain_t<3, 1>(hdr, done, table, nst, max_tiles, spin_limit, st);
    case 4: return launch_chain_t<4, 1>(hdr, done, table, nst, max_tiles, spin_limit, st);
    case 5: return launch_chain_t<5, 1>(hdr, done, table, nst, max_tiles, spin_limit, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace bin1
