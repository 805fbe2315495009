// A3: order-preserving reroute (UltraEP news article, section on the key
// designs: reroute splits the tokens of one native expert over its replicas;
// EPLB tutorial: the physical replica is looked up from the logical top-k ID).
//
// One wave per sub-block, the same sub-blocks the histogram counted.  The
// scanned workspace rows give, for every expert e, the rank range
// [run_e, next_e) its pairs of this sub-block occupy in flat (source rank,
// token, k) order.  If no quota boundary of e falls inside that range, every
// one of those pairs goes to the same instance (or to -1 beyond the last
// quota), so the wave first writes a per-expert code table in LDS: a physical
// slot, -1, or "split".  A plan has at most one boundary per replica, so split
// (sub-block, expert) cells are rare; only their pairs are ranked one by one:
// per split expert, a wave prefix sum over lanes of the counts in flat order.
// Everything else is one LDS read per pair, and the IDs stream in and the
// physical IDs stream out as non-temporal accesses: the first tiles load while
// the code table is built, later ones ahead of their use.  With
// E <= 256 the IDs come from the histogram's one-byte copy (16 bytes per lane
// per 1024-pair group) unless the sub-block holds padding or bad IDs, which
// read the int32 IDs (16 bytes per lane per 256-pair tile).
// Short waves (one sub-block each) keep HBM busier than persistent ones.
#include "ep_internal.h"

namespace ep {
namespace {

#ifndef EP_RR_UNROLL
#define EP_RR_UNROLL 4
#endif
#ifndef EP_RR_MAX_WAVES
#define EP_RR_MAX_WAVES 8
#endif
// groups of the byte copy in flight per wave: four (4096 pairs, 1 KiB per
// wave: the whole sub-block in the batched launches); one group ahead measured
// 15 % slower, eight (more registers) 8 % slower
#ifndef EP_RR_PF_GROUPS
#define EP_RR_PF_GROUPS 4
#endif
constexpr int kPfGroups = EP_RR_PF_GROUPS;

constexpr int32_t kSplit = (int32_t)0x80000000;

// first instance t in [0, n) of the list at `inst` whose cumulative end exceeds j
__device__ __forceinline__ int first_above(const int2 *inst, int n, int32_t j) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (j < inst[mid].x) hi = mid; else lo = mid + 1;
    }
    return lo;
}

// Split experts of a sub-block.  The first 64 live one per lane in registers
// (rank counter, current instance, its cumulative end and slot); their pairs
// carry the code kSplit | index.  Any further split expert (code kSplitLds)
// keeps its rank counter in LDS and is looked up by binary search.
struct SplitRegs {
    int32_t run;   // rank of the expert's next pair
    int32_t f, n;  // its instance list in the block table
    int32_t t;     // instance holding `run`
    int32_t end;   // cumulative end of instance t (INT32_MAX past the last)
    int32_t phys;  // slot of instance t (-1 past the last)
};

constexpr int32_t kSplitLds = (int32_t)(0x80000000u | 127u);

__device__ __forceinline__ bool is_split(int32_t c) { return c < -1; }

__device__ __forceinline__ void seek(SplitRegs &sr, const int2 *inst) {
    sr.t = first_above(inst + sr.f, sr.n, sr.run);
    sr.end = sr.t < sr.n ? inst[sr.f + sr.t].x : 0x7fffffff;
    sr.phys = sr.t < sr.n ? inst[sr.f + sr.t].y : -1;
}

// Rank the pairs of split experts in one group and replace their codes by the
// instance slot.  K consecutive pairs per lane; flat order is (lane, k), so
// the rank of (l, k) among pairs of one expert in the group is the number of
// its bits below lane l in the K column ballots plus its pairs in columns
// k' < k of lane l.  Loops once per distinct split expert present.
template <int K>
__device__ __forceinline__ void resolve_split(const int32_t (&x)[K], int32_t (&c)[K],
                                              SplitRegs &sr, const int32_t *rfirst,
                                              const int32_t *rcnt, const int2 *inst,
                                              int32_t *srun) {
    const uint64_t lt = lanemask_lt();
    const int lane = lane_id();
    uint32_t pend = 0;
#pragma unroll
    for (int k = 0; k < K; k++) pend |= (is_split(c[k]) ? 1u : 0u) << k;
    for (;;) {
        const uint64_t any = __ballot(pend != 0);
        if (any == 0) break;
        const int leader = __ffsll((long long)any) - 1;
        int32_t mc = 0, mx = 0;
#pragma unroll
        for (int k = K - 1; k >= 0; k--)
            if (pend & (1u << k)) { mc = c[k]; mx = x[k]; }
        const int32_t cc = __builtin_amdgcn_readlane(mc, leader);
        const int32_t y = __builtin_amdgcn_readlane(mx, leader);
        uint32_t hit = 0;
        int below = 0, tot = 0;
#pragma unroll
        for (int k = 0; k < K; k++) {
            const bool h = ((pend >> k) & 1u) && x[k] == y;
            hit |= (h ? 1u : 0u) << k;
            const uint64_t m = __ballot(h);
            below += __popcll(m & lt);
            tot += __popcll(m);
        }
        if (cc != kSplitLds) {
            const int idx = cc & 0x7f;
            const int32_t run = __builtin_amdgcn_readlane(sr.run, idx);
            const int32_t rend = __builtin_amdgcn_readlane(sr.end, idx);
            if (run + tot <= rend) {
                // the whole group sits in one instance
                const int32_t ph = __builtin_amdgcn_readlane(sr.phys, idx);
#pragma unroll
                for (int k = 0; k < K; k++)
                    if ((hit >> k) & 1u) c[k] = ph;
            } else {
                const int f = __builtin_amdgcn_readlane(sr.f, idx);
                const int n = __builtin_amdgcn_readlane(sr.n, idx);
                int r = run + below;
#pragma unroll
                for (int k = 0; k < K; k++) {
                    if ((hit >> k) & 1u) {
                        const int t = first_above(inst + f, n, r);
                        c[k] = t < n ? inst[f + t].y : -1;
                        r++;
                    }
                }
            }
            if (lane == idx) {
                sr.run = run + tot;
                if (sr.run >= sr.end) seek(sr, inst);
            }
        } else {
            const int32_t base = srun[y];
            const int f = rfirst[y], n = rcnt[y];
            int r = base + below;
#pragma unroll
            for (int k = 0; k < K; k++) {
                if ((hit >> k) & 1u) {
                    const int t = first_above(inst + f, n, r);
                    c[k] = t < n ? inst[f + t].y : -1;
                    r++;
                }
            }
            wave_lds_fence();
            if (lane == 0) srun[y] = base + tot;
            wave_lds_fence();
        }
        pend &= ~hit;
    }
}

// Reading the byte copy: at most 72 VGPRs (7 waves per SIMD; the compiler
// moves a few values of the rare split path to scratch), 5 % faster than the
// 78 it picks unbounded; at 8 waves (64 VGPRs) the spills cost more than the
// waves gain.  Reading int32 IDs the bound costs 2 %, so it is not set there.
template <int W, bool BYTES>
__global__ __launch_bounds__(W *kWave, BYTES ? 7 : 1) void reroute_kernel(
    const int32_t *__restrict__ ids, int64_t N, int32_t E, int32_t Phi, int32_t rho, int64_t sub,
    int64_t nsb, int64_t sps, int64_t nseg, const int32_t *__restrict__ ws, const int32_t *__restrict__ phy_quota,
    const int32_t *__restrict__ log2phy, const int32_t *__restrict__ logcnt,
    const int32_t *__restrict__ flags, const uint8_t *__restrict__ ids8, int64_t stride8,
    int32_t *__restrict__ out) {
    extern __shared__ __align__(16) unsigned char sh_raw[];
    int2 *inst = reinterpret_cast<int2 *>(sh_raw);                        // [Phi] (end, phys)
    int32_t *rfirst = reinterpret_cast<int32_t *>(inst + Phi);            // [E]
    int32_t *rcnt = rfirst + E;                                           // [E]
    int32_t *code_all = rcnt + E;                                         // [W][E]
    int32_t *srun_all = code_all + (size_t)W * E;                         // [W][E]
    int32_t *sidx_all = srun_all + (size_t)W * E;                         // [W][64]
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int p = blockIdx.y;
    const int E1 = E + 1;

    // --- route table of this plan: instances of each expert, cumulative quotas
    if (wave == 0) {
        int carry = 0;
        for (int c = 0; c < E; c += kWave) {
            const int e = c + lane;
            int n = 0;
            if (e < E) {
                n = logcnt[(int64_t)p * E + e];
                n = n < 0 ? 0 : (n > rho ? rho : n);
            }
            const int incl = wave_incl_scan_i32(n);
            if (e < E) {
                int start = carry + incl - n;
                if (start > Phi) start = Phi;
                if (start + n > Phi) n = Phi - start;
                rfirst[e] = start;
                rcnt[e] = n;
            }
            carry += __shfl(incl, kWave - 1);
        }
    }
    __syncthreads();
    // one thread per instance (an expert with many replicas would otherwise
    // chain two dependent global reads per instance): its slot and quota, then
    // per expert the running sum over its instances in LDS
    {
        const int total = E > 0 ? rfirst[E - 1] + rcnt[E - 1] : 0;
        for (int k = threadIdx.x; k < total; k += W * kWave) {
            // the expert owning instance k: the last e with rfirst[e] <= k
            int lo = 0, hi = E - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (rfirst[mid] <= k) lo = mid; else hi = mid - 1;
            }
            const int s = log2phy[((int64_t)p * E + lo) * rho + (k - rfirst[lo])];
            const bool ok = s >= 0 && s < Phi;
            inst[k] = make_int2(ok ? phy_quota[(int64_t)p * Phi + s] : 0, ok ? s : -1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += W * kWave) {
        const int f = rfirst[e], n = rcnt[e];
        int64_t acc = 0;
        for (int t = 0; t < n; t++) {
            acc += inst[f + t].x;
            inst[f + t].x = acc > 0x7fffffff ? 0x7fffffff : (acc < 0 ? 0 : (int32_t)acc);
        }
    }
    __syncthreads();

    const int64_t sb = (int64_t)blockIdx.x * W + wave;
    if (sb >= nsb) return;  // per-wave state below: no more block barriers
    int32_t *code = code_all + (size_t)wave * E;
    int32_t *srun = srun_all + (size_t)wave * E;
    int32_t *sidx = sidx_all + (size_t)wave * kWave;
    const int64_t begin = sb * sub;
    const int64_t end = (begin + sub < N) ? begin + sub : N;
    const int32_t *src = ids + (int64_t)p * N;
    int32_t *dst = out + (int64_t)p * N;
    const int64_t ntile = (end - begin) / (4 * kWave);  // whole 256-pair tiles
    const bool dst16 = (((uintptr_t)(dst + begin)) & 15) == 0;
    const bool src16 = (((uintptr_t)(src + begin)) & 15) == 0;
    const uint32_t *s8 = ids8 ? reinterpret_cast<const uint32_t *>(ids8 + (int64_t)p * stride8 + begin) : nullptr;
    const int32_t odd = ids8 ? flags[(int64_t)p * nsb + sb] : 1;
    // the first IDs load while the expert codes are set up: bytes when there
    // is a compact copy (a flagged sub-block discards them), else int32
    constexpr int U = EP_RR_UNROLL;
    static_assert(U == kGroupTiles, "one group of the byte copy per step");
    const int64_t ngroup = ntile / kGroupTiles;  // whole 1024-pair groups of the byte copy
    i32x4 pf[U];
    u32x4 pf8[kPfGroups];  // the next groups of the byte copy, in order
    const bool pf_bytes = BYTES && s8 && dst16 && ngroup > 0;
    const bool pf_words = !BYTES && dst16 && src16 && ntile >= U;
    if (pf_bytes) {
#pragma unroll
        for (int j = 0; j < kPfGroups; j++)
            if (j < ngroup) pf8[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(s8) + j * kWave + lane);
    }
    if (pf_words) {
#pragma unroll
        for (int u = 0; u < U; u++)
            pf[u] = __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(src + begin) + u * kWave + lane);
    }
    // --- per-expert code for this sub-block
    const SubPrefix pre = sub_prefix(ws, p, sb, nsb, sps, nseg, E1);
    int nsplit = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
        const int e = e0 + lane;
        int32_t cd = -1, run = 0;
        if (e < E) {
            run = pre.start(e);
            const int32_t nxt = pre.end(e);
            const int f = rfirst[e], n = rcnt[e];
            const int t = first_above(inst + f, n, run);
            if (nxt > run && t < n) cd = nxt <= inst[f + t].x ? inst[f + t].y : kSplit;
        }
        const bool sp = cd == kSplit;
        const uint64_t m = __ballot(sp);
        if (sp) {
            const int idx = nsplit + __popcll(m & lanemask_lt());
            if (idx < kWave) {
                cd = (int32_t)(0x80000000u | (uint32_t)idx);
                sidx[idx] = e;
            } else {
                cd = kSplitLds;
            }
        }
        nsplit += __popcll(m);
        if (e < E) { code[e] = cd; srun[e] = run; }
    }
    wave_lds_fence();
    SplitRegs sr{0, 0, 0, 0, 0x7fffffff, -1};
    if (lane < nsplit) {
        const int e = sidx[lane];
        sr.run = srun[e];
        sr.f = rfirst[e];
        sr.n = rcnt[e];
        seek(sr, inst);
    }

    const uint32_t uE = (uint32_t)E;
    int64_t g = begin;
    i32x4 *d4 = reinterpret_cast<i32x4 *>(dst + begin);
    // physical IDs of the 4 pairs of lane `lane` in tile tt
    auto emit = [&](int32_t (&x)[4], int64_t tt) {
        int32_t c[4];
        bool sp = false;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            c[k] = (uint32_t)x[k] < uE ? code[x[k]] : -1;
            sp |= is_split(c[k]);
        }
        if (__ballot(sp)) resolve_split<4>(x, c, sr, rfirst, rcnt, inst, srun);
        i32x4 o;
        o.x = c[0]; o.y = c[1]; o.z = c[2]; o.w = c[3];
        __builtin_nontemporal_store(o, d4 + tt * kWave + lane);
    };

    if (BYTES && s8 && dst16 && odd == 0) {
        // one-byte IDs: a whole group is one 16-byte load per lane (its 4 IDs
        // of each of the 4 tiles), kPfGroups groups ahead of their use.
        // Whole tiles after the last group hold their bytes in pair order.
        const u32x4 *g8 = reinterpret_cast<const u32x4 *>(s8);
        for (int64_t gi = 0; gi < ngroup; gi++) {
            const u32x4 wv = pf8[0];
#pragma unroll
            for (int j = 0; j + 1 < kPfGroups; j++) pf8[j] = pf8[j + 1];
            if (gi + kPfGroups < ngroup)
                pf8[kPfGroups - 1] = __builtin_nontemporal_load(g8 + (gi + kPfGroups) * kWave + lane);
            const uint32_t w[U] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int u = 0; u < U; u++) {
                int32_t x[4] = {(int32_t)(w[u] & 0xffu), (int32_t)((w[u] >> 8) & 0xffu),
                                (int32_t)((w[u] >> 16) & 0xffu), (int32_t)(w[u] >> 24)};
                emit(x, gi * U + u);
            }
        }
        for (int64_t tt = ngroup * U; tt < ntile; tt++) {
            const uint32_t w = __builtin_nontemporal_load(s8 + tt * kWave + lane);
            int32_t x[4] = {(int32_t)(w & 0xffu), (int32_t)((w >> 8) & 0xffu), (int32_t)((w >> 16) & 0xffu),
                            (int32_t)(w >> 24)};
            emit(x, tt);
        }
        g = begin + ntile * 4 * kWave;
    } else if (dst16 && src16) {
        // int32 IDs, 16 bytes per lane per tile, double-buffered likewise
        const i32x4 *s4 = reinterpret_cast<const i32x4 *>(src + begin);
        int64_t tt = 0;
        i32x4 nv[U];
        if (pf_words) {
#pragma unroll
            for (int u = 0; u < U; u++) nv[u] = pf[u];
        } else if (ntile >= U) {
#pragma unroll
            for (int u = 0; u < U; u++) nv[u] = __builtin_nontemporal_load(s4 + u * kWave + lane);
        }
        for (; tt + U <= ntile; tt += U) {
            i32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; u++) v[u] = nv[u];
            if (tt + 2 * U <= ntile) {
#pragma unroll
                for (int u = 0; u < U; u++) nv[u] = __builtin_nontemporal_load(s4 + (tt + U + u) * kWave + lane);
            }
#pragma unroll
            for (int u = 0; u < U; u++) {
                int32_t x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                emit(x, tt + u);
            }
        }
        for (; tt < ntile; tt++) {
            const i32x4 v = __builtin_nontemporal_load(s4 + tt * kWave + lane);
            int32_t x[4] = {v.x, v.y, v.z, v.w};
            emit(x, tt);
        }
        g = begin + ntile * 4 * kWave;
    }
    // one pair per lane for the rest (tail, or rows not 16-byte aligned)
    for (; g < end; g += kWave) {
        const int64_t i = g + lane;
        int32_t x[1] = {i < end ? src[i] : -1};
        int32_t c[1] = {(uint32_t)x[0] < uE ? code[x[0]] : -1};
        if (__ballot(is_split(c[0]))) resolve_split<1>(x, c, sr, rfirst, rcnt, inst, srun);
        if (i < end) dst[i] = c[0];
    }
}

int pick_waves(int E, int Phi) {
    for (int w = EP_RR_MAX_WAVES; w >= 1; w >>= 1)
        if (reroute_lds_bytes(E, Phi, w) <= kLdsPreferred) return w;
    return reroute_lds_bytes(E, Phi, 1) <= kLdsMax ? 1 : 0;
}

}  // namespace

size_t reroute_lds_bytes(int E, int Phi, int waves) {
    return (size_t)Phi * 8 + (size_t)E * 8 + (size_t)waves * (E * 8 + kWave * 4);
}

hipError_t launch_reroute(const int32_t *ids, int64_t N, int32_t P, const ep_layout_t &L,
                          const SubGeom &g, const int32_t *ws, const Compact &cp,
                          const int32_t *phy_quota, const int32_t *log2phy, const int32_t *logcnt,
                          int32_t *out, hipStream_t s) {
    const int64_t sub = g.sub, nsb = g.nsb, sps = g.sps, nseg = g.nseg;
    if (nsb == 0) return hipSuccess;
    const int E = L.num_experts, Phi = L.num_phys, rho = L.max_replicas;
    const int w = pick_waves(E, Phi);
    if (w == 0) return hipErrorInvalidValue;
    const size_t lds = reroute_lds_bytes(E, Phi, w);
    dim3 grid((unsigned)((nsb + w - 1) / w), (unsigned)P);
    const bool bytes = cp.bytes != nullptr;
#define EP_RR(WV, BY)                                                                                \
    hipLaunchKernelGGL((reroute_kernel<WV, BY>), grid, dim3(WV * kWave), lds, s, ids, N, E, Phi, rho, \
                       sub, nsb, sps, nseg, ws, phy_quota, log2phy, logcnt, cp.flags, cp.bytes,       \
                       cp.stride, out)
    if (bytes) {
        if (w == 8) EP_RR(8, true); else if (w == 4) EP_RR(4, true); else if (w == 2) EP_RR(2, true); else EP_RR(1, true);
    } else {
        if (w == 8) EP_RR(8, false); else if (w == 4) EP_RR(4, false); else if (w == 2) EP_RR(2, false); else EP_RR(1, false);
    }
#undef EP_RR
    return hipGetLastError();
}

}  // namespace ep
