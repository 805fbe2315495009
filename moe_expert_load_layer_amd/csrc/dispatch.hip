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
// rank gives the position directly.  Positions are unique, so the scattered
// writes of dispatch_src never collide.
#include "ep_internal.h"

namespace ep {
namespace {

struct alignas(16) GroupRank {
    uint64_t mask;
    int32_t run;
    int32_t pad;
};

template <int W>
__global__ __launch_bounds__(W *kWave) void dispatch_kernel(
    const int32_t *__restrict__ ids, int64_t N, int32_t E, int32_t Phi, int32_t rho, int64_t sub,
    int64_t nsb, const int32_t *__restrict__ ws, const int32_t *__restrict__ phy_quota,
    const int32_t *__restrict__ log2phy, const int32_t *__restrict__ logcnt,
    int32_t *__restrict__ slot_offsets, int32_t *__restrict__ dpos, int32_t *__restrict__ dsrc) {
    extern __shared__ __align__(16) unsigned char sh_raw[];
    GroupRank *st_all = reinterpret_cast<GroupRank *>(sh_raw);              // [W][E]
    int2 *inst = reinterpret_cast<int2 *>(st_all + (size_t)W * E);          // [Phi] (end, off - Q)
    int32_t *soff = reinterpret_cast<int32_t *>(inst + Phi);                // [Phi + 1]
    int32_t *rfirst = soff + Phi + 1;                                       // [E]
    int32_t *rcnt = rfirst + E;                                             // [E]
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
    GroupRank *st = st_all + (size_t)wave * E;
    const int32_t *row0 = ws + ((int64_t)p * (nsb + 1) + sb) * E1;
    for (int e = lane; e < E; e += kWave) st[e] = GroupRank{0ull, row0[e], 0};
    wave_lds_fence();

    const int64_t begin = sb * sub;
    const int64_t end = (begin + sub < N) ? begin + sub : N;
    const int32_t *src = ids + (int64_t)p * N;
    int32_t *pos_out = dpos + (int64_t)p * N;
    int32_t *src_out = dsrc + (int64_t)p * N;
    const uint64_t lt = lanemask_lt();
    const uint64_t bit = 1ull << lane;
    const uint32_t uE = (uint32_t)E;
    constexpr int U = 4;
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
            GroupRank cur{0ull, 0, 0};
            if (valid) cur = st[x];
            wave_lds_fence();
            int32_t pos = -1;
            if (valid) {
                const uint64_t below = cur.mask & lt;
                if (below == 0) st[x] = GroupRank{0ull, cur.run + (int32_t)__popcll(cur.mask), 0};
                const int32_t j = cur.run + (int32_t)__popcll(below);
                const int f = rfirst[x], n = rcnt[x];
                int lo = 0, hi = n;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (j < inst[f + mid].x) hi = mid; else lo = mid + 1;
                }
                if (lo < n && inst[f + lo].y != (int32_t)0x80000000) pos = j + inst[f + lo].y;
            }
            const int64_t i = g + u * kWave + lane;
            if (i < end) {
                pos_out[i] = pos;
                if (pos >= 0 && pos < N) src_out[pos] = (int32_t)i;
            }
            wave_lds_fence();
        }
    }
    // positions past the plan's total quota hold no pair
    const int64_t tail = soff[Phi] > begin ? soff[Phi] : begin;
    for (int64_t i = tail + lane; i < end; i += kWave) src_out[i] = -1;
}

int pick_dispatch_waves(int E, int Phi) {
    for (int w = 4; w >= 1; w >>= 1)
        if (dispatch_lds_bytes(E, Phi, w) <= 65536) return w;
    return 0;
}

}  // namespace

size_t dispatch_lds_bytes(int E, int Phi, int waves) {
    return (size_t)waves * E * sizeof(GroupRank) + (size_t)Phi * 8 + (size_t)(Phi + 1) * 4 + (size_t)E * 8;
}

hipError_t launch_dispatch(const int32_t *ids, int64_t N, int32_t P, const ep_layout_t &L, int64_t sub,
                           int64_t nsb, const int32_t *ws, const int32_t *phy_quota,
                           const int32_t *log2phy, const int32_t *logcnt, int32_t *slot_offsets,
                           int32_t *dpos, int32_t *dsrc, hipStream_t s) {
    const int E = L.num_experts, Phi = L.num_phys, rho = L.max_replicas;
    const int w = pick_dispatch_waves(E, Phi);
    if (w == 0) return hipErrorInvalidValue;
    const size_t lds = dispatch_lds_bytes(E, Phi, w);
    // at least one block per plan so the slot offsets are always written
    const int64_t nblk = nsb > 0 ? (nsb + w - 1) / w : 1;
    dim3 grid((unsigned)nblk, (unsigned)P);
    switch (w) {
        case 4:
            hipLaunchKernelGGL(dispatch_kernel<4>, grid, dim3(4 * kWave), lds, s, ids, N, E, Phi, rho,
                               sub, nsb, ws, phy_quota, log2phy, logcnt, slot_offsets, dpos, dsrc);
            break;
        case 2:
            hipLaunchKernelGGL(dispatch_kernel<2>, grid, dim3(2 * kWave), lds, s, ids, N, E, Phi, rho,
                               sub, nsb, ws, phy_quota, log2phy, logcnt, slot_offsets, dpos, dsrc);
            break;
        default:
            hipLaunchKernelGGL(dispatch_kernel<1>, grid, dim3(kWave), lds, s, ids, N, E, Phi, rho, sub,
                               nsb, ws, phy_quota, log2phy, logcnt, slot_offsets, dpos, dsrc);
            break;
    }
    return hipGetLastError();
}

}  // namespace ep
