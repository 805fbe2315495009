// A1: exact per-expert load after the gate (UltraEP news article, section on
// the key designs: the global load is read after the gate, before planning).
//
// Two kernels:
//   hist_kernel  one wave per sub-block of consecutive pairs; counts into a
//                wave-private LDS histogram (E bins + one bin for IDs >= E)
//                with LDS integer atomics, then writes the row to the
//                workspace.  The IDs stream in as 16-byte loads.
//   scan_kernel  per (plan, 64 experts): turns the sub-block rows into
//                exclusive per-expert offsets in place (what the reroute needs
//                for a stable order) and writes load[p][e] = total and the
//                plan's status word.
// Integer counts only, so the result does not depend on atomic order.
#include "ep_internal.h"

namespace ep {
namespace {

#ifndef EP_HIST_WAVES
#define EP_HIST_WAVES 4
#endif
#ifndef EP_HIST_UNROLL
#define EP_HIST_UNROLL 4
#endif
constexpr int kHistWaves = EP_HIST_WAVES;

__global__ __launch_bounds__(kHistWaves * kWave) void hist_kernel(
    const int32_t *__restrict__ ids, int64_t N, int32_t E, int64_t sub, int64_t nsb,
    int32_t *__restrict__ ws) {
    extern __shared__ int32_t sh_hist[];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int E1 = E + 1;
    int32_t *h = sh_hist + wave * E1;
    const int64_t sb = (int64_t)blockIdx.x * kHistWaves + wave;
    const int p = blockIdx.y;
    if (sb >= nsb) return;  // wave-private LDS: no block barrier below

    for (int e = lane; e < E1; e += kWave) h[e] = 0;
    wave_lds_fence();

    const int64_t begin = sb * sub;
    const int64_t end = (begin + sub < N) ? begin + sub : N;
    const int32_t *src = ids + (int64_t)p * N;
    const uint32_t uE = (uint32_t)E;
    int nbad = 0;

    auto count = [&](int32_t v) {
        if ((uint32_t)v < uE) {
            atomicAdd(&h[v], 1);
        } else if (v >= E) {
            nbad++;
        }
    };

    int64_t i = begin;
    // 16-byte path: the plan row and sub-block start are 16-byte aligned
    if (((uintptr_t)(src + begin) & 15) == 0) {
        const int64_t nvec = (end - begin) / 4;
        const i32x4 *v4 = reinterpret_cast<const i32x4 *>(src + begin);
        constexpr int U = EP_HIST_UNROLL;
        int64_t k = lane;
        for (; k + (U - 1) * kWave < nvec; k += U * kWave) {
            i32x4 x[U];
#pragma unroll
            for (int u = 0; u < U; u++) x[u] = __builtin_nontemporal_load(v4 + k + u * kWave);
#pragma unroll
            for (int u = 0; u < U; u++) {
                count(x[u].x); count(x[u].y); count(x[u].z); count(x[u].w);
            }
        }
        for (; k < nvec; k += kWave) {
            const i32x4 x = __builtin_nontemporal_load(v4 + k);
            count(x.x); count(x.y); count(x.z); count(x.w);
        }
        i = begin + nvec * 4;
    }
    for (int64_t j = i + lane; j < end; j += kWave) count(src[j]);
    if (nbad) atomicAdd(&h[E], nbad);
    wave_lds_fence();

    int32_t *row = ws + ((int64_t)p * (nsb + 1) + sb) * E1;
    for (int e = lane; e < E1; e += kWave) row[e] = h[e];
}

constexpr int kScanWaves = 16;
constexpr int kScanUnroll = 8;

// Workspace rows per plan: nsb sub-block rows, then one row of per-expert
// totals (the plan's load), which lets the reroute skip ranking pairs of an
// expert whose single instance takes all of its pairs.
__global__ __launch_bounds__(kScanWaves * kWave) void scan_kernel(
    int32_t *__restrict__ ws, int64_t nsb, int32_t E, int32_t *__restrict__ load,
    uint32_t *__restrict__ status) {
    __shared__ int32_t part[kScanWaves][kWave];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int E1 = E + 1;
    const int p = blockIdx.y;
    const int col = blockIdx.x * kWave + lane;
    int32_t *base = ws + (int64_t)p * (nsb + 1) * E1;
    const int64_t seg = (nsb + kScanWaves - 1) / kScanWaves;
    const int64_t b0 = wave * seg < nsb ? wave * seg : nsb;
    const int64_t b1 = (b0 + seg < nsb) ? b0 + seg : nsb;
    const bool on = col < E1;

    int32_t sum = 0;
    if (on) {
        int64_t b = b0;
        for (; b + kScanUnroll <= b1; b += kScanUnroll) {
            int32_t c[kScanUnroll];
#pragma unroll
            for (int u = 0; u < kScanUnroll; u++) c[u] = base[(b + u) * E1 + col];
#pragma unroll
            for (int u = 0; u < kScanUnroll; u++) sum += c[u];
        }
        for (; b < b1; b++) sum += base[b * E1 + col];
    }
    part[wave][lane] = sum;
    __syncthreads();
    int32_t run = 0, total = 0;
    for (int w = 0; w < kScanWaves; w++) {
        if (w < wave) run += part[w][lane];
        total += part[w][lane];
    }
    if (on) {
        int64_t b = b0;
        for (; b + kScanUnroll <= b1; b += kScanUnroll) {
            int32_t c[kScanUnroll];
#pragma unroll
            for (int u = 0; u < kScanUnroll; u++) c[u] = base[(b + u) * E1 + col];
#pragma unroll
            for (int u = 0; u < kScanUnroll; u++) {
                base[(b + u) * E1 + col] = run;
                run += c[u];
            }
        }
        for (; b < b1; b++) {
            const int32_t c = base[b * E1 + col];
            base[b * E1 + col] = run;
            run += c;
        }
        if (wave == 0) {
            base[nsb * E1 + col] = total;
            if (col < E) load[(int64_t)p * E + col] = total;
            else status[p] = total > 0 ? (uint32_t)EP_STATUS_BAD_ID : 0u;
        }
    }
}

}  // namespace

hipError_t launch_histogram(const int32_t *ids, int64_t N, int32_t P, int32_t E, int64_t sub,
                            int64_t nsb, int32_t *ws, int32_t *load, uint32_t *status,
                            hipStream_t s) {
    if (nsb > 0) {
        dim3 grid((unsigned)((nsb + kHistWaves - 1) / kHistWaves), (unsigned)P);
        const size_t lds = (size_t)kHistWaves * (E + 1) * sizeof(int32_t);
        hipLaunchKernelGGL(hist_kernel, grid, dim3(kHistWaves * kWave), lds, s, ids, N, E, sub,
                           nsb, ws);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    dim3 g2((unsigned)((E + 1 + kWave - 1) / kWave), (unsigned)P);
    hipLaunchKernelGGL(scan_kernel, g2, dim3(kScanWaves * kWave), 0, s, ws, nsb, E, load, status);
    return hipGetLastError();
}

}  // namespace ep
