// Dispatch layout for the token all-to-all (EPLB tutorial, EPLB / DeepEP
// section: dispatch sends each pair to its physical replica, combine gathers
// the results back to the logical expert).  The pairs of a plan are laid out
// physical-slot-major: slot s owns positions [off_s, off_s + quota_s), off
// the exclusive prefix of the quotas in slot order, and the j-th pair of
// expert e, served by instance s whose quota range starts at Q, goes to
// position off_s + (j - Q).  With quotas that cover the loads this is the
// stable counting sort of the pairs by physical slot.
//
// One wave per sub-block (the histogram's).  Every pair needs its rank among
// the pairs of its expert, so each 64-pair group is ranked with an LDS bit
// mask per expert (each lane ORs its bit, counts the bits below it) plus a
// per-expert running count started from the scanned workspace row.  The block
// lays out per instance (cumulative end, off_s - Q) so a binary search on the
// rank gives the position directly.  Positions are unique, so the writes of
// dispatch_src never collide.
//
// dispatch_src is written through LDS: each wave stages the in-sub-block index
// of every pair at (expert's offset within the sub-block + its rank k there),
// then walks the experts in order; the pairs of one expert occupy consecutive
// positions (one run per instance it spans), so the stores are coalesced
// runs instead of 4-byte scatters.  Sub-blocks too large for the staging
// buffer scatter directly.
#include "ep_internal.h"

namespace ep {
namespace {

// Per-expert state of a wave's sub-block: ranks come from the bit mask of the
// current 64-pair group plus the count of earlier groups.
struct CellState {
    uint64_t mask;
    int32_t k;     // pairs of the expert seen so far in this sub-block
    int32_t off;   // staging offset of the expert's pairs (staged layout)
};

// Where an expert's pairs of one sub-block go: staging offset, first rank,
// count, and the position shift of the one instance that takes all of them
// (kSplitCell if they cross a quota boundary, kNoCell if none is placed).
struct CellInfo {
    int32_t off;
    int32_t run;
    int32_t cnt;
    int32_t delta;
};

constexpr int32_t kSplitCell = (int32_t)0x80000000;
constexpr int32_t kNoCell = (int32_t)0x80000001;

__device__ __forceinline__ int32_t position_of(const int2 *inst, int f, int n, int32_t j) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (j < inst[f + mid].x) hi = mid; else lo = mid + 1;
    }
    if (lo < n && inst[f + lo].y != (int32_t)0x80000000) return j + inst[f + lo].y;
    return -1;
}

template <int W, bool STAGED>
__global__ __launch_bounds__(W *kWave) void dispatch_kernel(
    const int32_t *__restrict__ ids, int64_t N, int32_t E, int32_t Phi, int32_t rho, int64_t sub,
    int64_t nsb, int64_t sps, int64_t nseg, const int32_t *__restrict__ ws, const int32_t *__restrict__ phy_quota,
    const int32_t *__restrict__ log2phy, const int32_t *__restrict__ logcnt,
    int32_t *__restrict__ slot_offsets, int32_t *__restrict__ dpos, int32_t *__restrict__ dsrc) {
    extern __shared__ __align__(16) unsigned char sh_raw[];
    CellState *st_all = reinterpret_cast<CellState *>(sh_raw);             // [W][E]
    CellInfo *ci_all = reinterpret_cast<CellInfo *>(st_all + (size_t)W * E); // [W][E]
    int2 *inst = reinterpret_cast<int2 *>(ci_all + (size_t)W * E);          // [Phi] (end, off - Q)
    int32_t *soff = reinterpret_cast<int32_t *>(inst + Phi);                // [Phi + 1]
    int32_t *rfirst = soff + Phi + 1;                                       // [E]
    int32_t *rcnt = rfirst + E;                                             // [E]
    uint16_t *stage_all = reinterpret_cast<uint16_t *>(rcnt + E);           // [W][sub] if STAGED
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int p = blockIdx.y;
    const int E1 = E + 1;

    if (wave == 0) {
        // slot offsets: exclusive prefix of the quotas in slot order
        int carry = 0;
        for (int c = 0; c < Phi; c += kWave) {
            const int s = c + lane;
            const int q = s < Phi ? phy_quota[(int64_t)p * Phi + s] : 0;
            const int incl = wave_incl_scan_i32(q);
            if (s < Phi) soff[s] = carry + incl - q;
            carry += __shfl(incl, kWave - 1);
        }
        if (lane == 0) soff[Phi] = carry;
        // instance lists of the experts
        carry = 0;
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
    for (int e = threadIdx.x; e < E; e += W * kWave) {
        const int f = rfirst[e], n = rcnt[e];
        const int32_t *row = log2phy + ((int64_t)p * E + e) * rho;
        int32_t acc = 0;
        for (int t = 0; t < n; t++) {
            const int s = row[t];
            const bool ok = s >= 0 && s < Phi;
            const int32_t q = ok ? phy_quota[(int64_t)p * Phi + s] : 0;
            inst[f + t] = make_int2(acc + q, ok ? soff[s] - acc : 0x80000000);
            acc += q;
        }
    }
    if (blockIdx.x == 0)
        for (int s = threadIdx.x; s <= Phi; s += W * kWave) slot_offsets[(int64_t)p * (Phi + 1) + s] = soff[s];
    __syncthreads();

    const int64_t sb = (int64_t)blockIdx.x * W + wave;
    if (sb >= nsb) return;  // per-wave state below: no more block barriers
    CellState *st = st_all + (size_t)wave * E;
    CellInfo *ci = ci_all + (size_t)wave * E;
    uint16_t *stage = stage_all + (size_t)wave * (STAGED ? sub : 0);
    const SubPrefix pre = sub_prefix(ws, p, sb, nsb, sps, nseg, E1);
    {
        int carry = 0;
        for (int c = 0; c < E; c += kWave) {
            const int e = c + lane;
            int32_t run = 0, cnt = 0, delta = kNoCell;
            if (e < E) {
                run = pre.start(e);
                cnt = pre.end(e) - run;
                const int f = rfirst[e], n = rcnt[e];
                int lo = 0, hi = n;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (run < inst[f + mid].x) hi = mid; else lo = mid + 1;
                }
                if (cnt > 0 && lo < n && inst[f + lo].y != (int32_t)0x80000000)
                    delta = run + cnt <= inst[f + lo].x ? inst[f + lo].y : kSplitCell;
                else if (cnt > 0 && lo < n)
                    delta = kSplitCell;
            }
            const int incl = wave_incl_scan_i32(cnt);
            if (e < E) {
                ci[e] = CellInfo{carry + incl - cnt, run, cnt, delta};
                st[e] = CellState{0ull, 0, carry + incl - cnt};
            }
            carry += __shfl(incl, kWave - 1);
        }
    }
    wave_lds_fence();

    const int64_t begin = sb * sub;
    const int64_t end = (begin + sub < N) ? begin + sub : N;
    const int32_t *src = ids + (int64_t)p * N;
    int32_t *pos_out = dpos + (int64_t)p * N;
    int32_t *src_out = dsrc + (int64_t)p * N;
    const uint64_t lt = lanemask_lt();
    const uint64_t bit = 1ull << lane;
    const uint32_t uE = (uint32_t)E;
    constexpr int U = 8;
    for (int64_t g = begin; g < end; g += U * kWave) {
        int32_t v[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t i = g + u * kWave + lane;
            v[u] = i < end ? __builtin_nontemporal_load(src + i) : -1;
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int32_t x = v[u];
            const bool valid = (uint32_t)x < uE;
            if (valid) atomicOr(reinterpret_cast<unsigned long long *>(&st[x].mask), bit);
            wave_lds_fence();
            CellState cur{0ull, 0, 0};
            if (valid) cur = st[x];
            wave_lds_fence();
            const int64_t i = g + u * kWave + lane;
            int32_t pos = -1;
            if (valid) {
                const uint64_t below = cur.mask & lt;
                if (below == 0) st[x] = CellState{0ull, cur.k + (int32_t)__popcll(cur.mask), cur.off};
                const int32_t k = cur.k + (int32_t)__popcll(below);
                const CellInfo cell = ci[x];
                const int32_t j = cell.run + k;
                if (cell.delta == kSplitCell) pos = position_of(inst, rfirst[x], rcnt[x], j);
                else if (cell.delta != kNoCell) pos = j + cell.delta;
                if (STAGED) stage[cur.off + k] = (uint16_t)(i - begin);
                else if (pos >= 0 && pos < N) src_out[pos] = (int32_t)i;
            }
            if (i < end) pos_out[i] = pos;
            wave_lds_fence();
        }
    }
    if (STAGED) {
        // experts in order, 64 at a time: each expert's staged pairs go to
        // consecutive positions (per instance), written as coalesced runs
        for (int c = 0; c < E; c += kWave) {
            const int e = c + lane;
            CellInfo mine{0, 0, 0, kNoCell};
            if (e < E) mine = ci[e];
            const int last = (E - c) < kWave ? E - c : kWave;
            for (int l = 0; l < last; l++) {
                const int32_t cnt = __builtin_amdgcn_readlane(mine.cnt, l);
                const int32_t delta = __builtin_amdgcn_readlane(mine.delta, l);
                if (cnt == 0 || delta == kNoCell) continue;
                const int32_t off = __builtin_amdgcn_readlane(mine.off, l);
                const int32_t run = __builtin_amdgcn_readlane(mine.run, l);
                for (int32_t t = lane; t < cnt; t += kWave) {
                    const int32_t j = run + t;
                    int32_t pos = -1;
                    if (delta == kSplitCell) pos = position_of(inst, rfirst[c + l], rcnt[c + l], j);
                    else if (delta != kNoCell) pos = j + delta;
                    if (pos >= 0 && pos < N) src_out[pos] = (int32_t)(begin + stage[off + t]);
                }
            }
        }
    }
    // positions past the plan's total quota hold no pair
    const int64_t tail = soff[Phi] > begin ? soff[Phi] : begin;
    for (int64_t i = tail + lane; i < end; i += kWave) src_out[i] = -1;
}

int pick_dispatch_waves(int E, int Phi, int64_t stage) {
    for (int w = 4; w >= 1; w >>= 1)
        if (dispatch_lds_bytes(E, Phi, w, stage) <= 65536) return w;
    return 0;
}

}  // namespace

size_t dispatch_lds_bytes(int E, int Phi, int waves, int64_t stage_pairs) {
    return (size_t)waves * E * (sizeof(CellState) + sizeof(CellInfo)) + (size_t)Phi * 8 +
           (size_t)(Phi + 1) * 4 + (size_t)E * 8 + (size_t)waves * stage_pairs * 2;
}

hipError_t launch_dispatch(const int32_t *ids, int64_t N, int32_t P, const ep_layout_t &L,
                           const SubGeom &g, const int32_t *ws, const int32_t *phy_quota,
                           const int32_t *log2phy, const int32_t *logcnt, int32_t *slot_offsets,
                           int32_t *dpos, int32_t *dsrc, hipStream_t s) {
    const int64_t sub = g.sub, nsb = g.nsb, sps = g.sps, nseg = g.nseg;
    const int E = L.num_experts, Phi = L.num_phys, rho = L.max_replicas;
    // stage through LDS when a sub-block's pair indices fit (16-bit, 1 or 2 waves)
    int w = sub <= 65536 ? pick_dispatch_waves(E, Phi, sub) : 0;
    const bool staged = w > 0;
    if (!staged) w = pick_dispatch_waves(E, Phi, 0);
    if (w == 0) return hipErrorInvalidValue;
    const size_t lds = dispatch_lds_bytes(E, Phi, w, staged ? sub : 0);
    // at least one block per plan so the slot offsets are always written
    const int64_t nblk = nsb > 0 ? (nsb + w - 1) / w : 1;
    dim3 grid((unsigned)nblk, (unsigned)P);
#define EP_DISPATCH(WV, ST)                                                                        \
    hipLaunchKernelGGL((dispatch_kernel<WV, ST>), grid, dim3(WV * kWave), lds, s, ids, N, E, Phi, rho, \
                       sub, nsb, sps, nseg, ws, phy_quota, log2phy, logcnt, slot_offsets, dpos, dsrc)
    if (staged) {
        if (w == 4) EP_DISPATCH(4, true); else if (w == 2) EP_DISPATCH(2, true); else EP_DISPATCH(1, true);
    } else {
        if (w == 4) EP_DISPATCH(4, false); else if (w == 2) EP_DISPATCH(2, false); else EP_DISPATCH(1, false);
    }
#undef EP_DISPATCH
    return hipGetLastError();
}

}  // namespace ep
