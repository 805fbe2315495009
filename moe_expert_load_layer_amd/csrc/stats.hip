// A5: balance statistics (UltraEP digest, "Reported results": the most loaded
// rank relative to the average load; EPLB tutorial: balancedness = mean / max).
// One workgroup per plan: per-rank loads before (native placement) and after
// (sum of the quotas on the rank), their maxima, the total and the replicas in
// use; imbalance = max * R / total as one correctly rounded double division.
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kStatThreads = 256;

__global__ __launch_bounds__(kStatThreads) void stats_kernel(
    const int32_t *__restrict__ load, const int32_t *__restrict__ quota, int32_t E, int32_t R,
    int32_t Phi, Tables T, int64_t *__restrict__ stats, double *__restrict__ imb,
    int32_t *__restrict__ rank_load) {
    __shared__ int64_t red[4][kStatThreads / kWave];
    const int p = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t *lp = load + (int64_t)p * E;
    const int32_t *qp = quota + (int64_t)p * Phi;
    int64_t mb = 0, ma = 0, used = 0, tot = 0;
    for (int r = tid; r < R; r += kStatThreads) {
        const int f = T.rank_first[r], l = T.rank_first[r + 1], nat = T.rank_nat[r];
        int64_t before = 0, after = 0;
        for (int s = f; s < l; s++) {
            const int32_t q = qp[s];
            if (s < f + nat) before += lp[T.slot_home[s]];
            else if (q > 0) used++;
            after += q;
        }
        if (rank_load) {
            rank_load[(int64_t)p * 2 * R + r] = (int32_t)before;
            rank_load[(int64_t)p * 2 * R + R + r] = (int32_t)after;
        }
        mb = before > mb ? before : mb;
        ma = after > ma ? after : ma;
    }
    for (int e = tid; e < E; e += kStatThreads) tot += lp[e];
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) {
        const int64_t a = (int64_t)shfl_xor_u64((uint64_t)mb, m);
        const int64_t b = (int64_t)shfl_xor_u64((uint64_t)ma, m);
        mb = a > mb ? a : mb;
        ma = b > ma ? b : ma;
        used += (int64_t)shfl_xor_u64((uint64_t)used, m);
        tot += (int64_t)shfl_xor_u64((uint64_t)tot, m);
    }
    const int wave = tid / kWave;
    if (lane_id() == 0) { red[0][wave] = mb; red[1][wave] = ma; red[2][wave] = used; red[3][wave] = tot; }
    __syncthreads();
    if (tid == 0) {
        int64_t MB = 0, MA = 0, U = 0, TOT = 0;
        for (int w = 0; w < kStatThreads / kWave; w++) {
            MB = red[0][w] > MB ? red[0][w] : MB;
            MA = red[1][w] > MA ? red[1][w] : MA;
            U += red[2][w];
            TOT += red[3][w];
        }
        int64_t *st = stats + (int64_t)p * 4;
        st[0] = MB; st[1] = MA; st[2] = TOT; st[3] = U;
        imb[(int64_t)p * 2 + 0] = TOT > 0 ? (double)(MB * (int64_t)R) / (double)TOT : 1.0;
        imb[(int64_t)p * 2 + 1] = TOT > 0 ? (double)(MA * (int64_t)R) / (double)TOT : 1.0;
    }
}

}  // namespace

hipError_t launch_stats(const int32_t *load, const int32_t *phy_quota, int32_t P,
                        const ep_layout_t &L, int64_t *stats, double *imbalance,
                        int32_t *rank_load, hipStream_t s) {
    hipLaunchKernelGGL(stats_kernel, dim3((unsigned)P), dim3(kStatThreads), 0, s, load, phy_quota,
                       L.num_experts, L.num_ranks, L.num_phys, tables_of(L), stats, imbalance,
                       rank_load);
    return hipGetLastError();
}

}  // namespace ep
