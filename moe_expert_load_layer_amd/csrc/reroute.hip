// A3: order-preserving reroute (UltraEP news article, section on the key
// designs: reroute splits the tokens of one native expert over its replicas;
// EPLB tutorial: the physical replica is looked up from the logical top-k ID).
//
// One wave per sub-block, the same sub-blocks the histogram counted.  The
// scanned workspace row gives, for every expert, how many of its pairs come
// before the sub-block.  Inside the sub-block the wave walks 64 pairs at a time
// in flat order; the stable rank of a pair among equal IDs of the group comes
// from an LDS bit mask per expert (each lane ORs its bit, then counts the bits
// below it), so no atomic order is involved.  The group leader of each expert
// advances that expert's running count.  The rank j then selects the instance
// whose cumulative quota range holds j (binary search over the expert's
// instances, which the block lays out in LDS from log2phy and phy_quota).
#include "ep_internal.h"

namespace ep {
namespace {

template <int W>
__global__ __launch_bounds__(W *kWave) void reroute_kernel(
    const int32_t *__restrict__ ids, int64_t N, int32_t E, int32_t Phi, int32_t rho, int64_t sub,
    int64_t nsb, const int32_t *__restrict__ ws, const int32_t *__restrict__ phy_quota,
    const int32_t *__restrict__ log2phy, const int32_t *__restrict__ logcnt,
    int32_t *__restrict__ out) {
    extern __shared__ __align__(16) unsigned char sh_raw[];
    uint64_t *mask_all = reinterpret_cast<uint64_t *>(sh_raw);               // [W][E]
    int32_t *run_all = reinterpret_cast<int32_t *>(mask_all + (size_t)W * E);  // [W][E]
    int32_t *rfirst = run_all + (size_t)W * E;                                 // [E]
    int32_t *rcnt = rfirst + E;                                                // [E]
    int32_t *iend = rcnt + E;                                                  // [Phi]
    int32_t *iphys = iend + Phi;                                               // [Phi]
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int p = blockIdx.y;

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
                int nn = n;
                if (start >= Phi) { start = Phi; nn = 0; }
                else if (start + nn > Phi) nn = Phi - start;
                rfirst[e] = start;
                rcnt[e] = nn;
            }
            carry += __shfl(incl, kWave - 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += W * kWave) {
        const int f = rfirst[e], n = rcnt[e];
        const int32_t *row = log2phy + ((int64_t)p * E + e) * rho;
        int64_t acc = 0;
        for (int t = 0; t < n; t++) {
            const int s = row[t];
            const bool ok = s >= 0 && s < Phi;
            acc += ok ? phy_quota[(int64_t)p * Phi + s] : 0;
            iend[f + t] = acc > 0x7fffffff ? 0x7fffffff : (acc < 0 ? 0 : (int32_t)acc);
            iphys[f + t] = ok ? s : -1;
        }
    }
    __syncthreads();

    const int64_t sb = (int64_t)blockIdx.x * W + wave;
    if (sb >= nsb) return;  // per-wave state below: no more block barriers
    uint64_t *mask = mask_all + (size_t)wave * E;
    int32_t *run = run_all + (size_t)wave * E;
    const int32_t *row = ws + ((int64_t)p * nsb + sb) * (E + 1);
    for (int e = lane; e < E; e += kWave) { run[e] = row[e]; mask[e] = 0; }
    wave_lds_fence();

    const int64_t begin = sb * sub;
    const int64_t end = (begin + sub < N) ? begin + sub : N;
    const int32_t *src = ids + (int64_t)p * N;
    int32_t *dst = out + (int64_t)p * N;
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
            if (valid) atomicOr(reinterpret_cast<unsigned long long *>(&mask[x]), bit);
            wave_lds_fence();
            uint64_t m = 0;
            int32_t base = 0;
            if (valid) { m = mask[x]; base = run[x]; }
            wave_lds_fence();
            const uint64_t below = m & lt;
            int32_t phys = -1;
            if (valid) {
                if (below == 0) { run[x] = base + (int32_t)__popcll(m); mask[x] = 0; }
                const int32_t j = base + (int32_t)__popcll(below);
                const int f = rfirst[x], n = rcnt[x];
                int lo = 0, hi = n;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (j < iend[f + mid]) hi = mid; else lo = mid + 1;
                }
                phys = lo < n ? iphys[f + lo] : -1;
            }
            const int64_t i = g + u * kWave + lane;
            if (i < end) __builtin_nontemporal_store(phys, dst + i);
            wave_lds_fence();
        }
    }
}

int pick_waves(int E, int Phi) {
    for (int w = 4; w >= 1; w >>= 1)
        if (reroute_lds_bytes(E, Phi, w) <= 65536) return w;
    return 0;
}

}  // namespace

size_t reroute_lds_bytes(int E, int Phi, int waves) {
    return (size_t)waves * E * 12 + (size_t)E * 8 + (size_t)Phi * 8;
}

hipError_t launch_reroute(const int32_t *ids, int64_t N, int32_t P, const ep_layout_t &L,
                          int64_t sub, int64_t nsb, const int32_t *ws, const int32_t *phy_quota,
                          const int32_t *log2phy, const int32_t *logcnt, int32_t *out,
                          hipStream_t s) {
    if (nsb == 0) return hipSuccess;
    const int E = L.num_experts, Phi = L.num_phys, rho = L.max_replicas;
    const int w = pick_waves(E, Phi);
    if (w == 0) return hipErrorInvalidValue;
    const size_t lds = reroute_lds_bytes(E, Phi, w);
    dim3 grid((unsigned)((nsb + w - 1) / w), (unsigned)P);
    switch (w) {
        case 4:
            hipLaunchKernelGGL(reroute_kernel<4>, grid, dim3(4 * kWave), lds, s, ids, N, E, Phi,
                               rho, sub, nsb, ws, phy_quota, log2phy, logcnt, out);
            break;
        case 2:
            hipLaunchKernelGGL(reroute_kernel<2>, grid, dim3(2 * kWave), lds, s, ids, N, E, Phi,
                               rho, sub, nsb, ws, phy_quota, log2phy, logcnt, out);
            break;
        default:
            hipLaunchKernelGGL(reroute_kernel<1>, grid, dim3(kWave), lds, s, ids, N, E, Phi, rho,
                               sub, nsb, ws, phy_quota, log2phy, logcnt, out);
            break;
    }
    return hipGetLastError();
}

}  // namespace ep
