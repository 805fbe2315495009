// A1: exact per-expert load after the gate (UltraEP news article, section on
// the key designs: the global load is read after the gate, before planning).
//
// Two kernels:
//   hist_kernel  one workgroup per segment of kSegSubs consecutive
//                sub-blocks, one wave per sub-block; each wave counts into
//                its own LDS histogram (E bins + one bin for IDs >= E) with
//                LDS integer atomics, the IDs streaming in as 16-byte loads.
//                After a barrier each wave stores its sub-block's in-segment
//                prefix (the sum of the lower waves' histograms) and the last
//                wave also the segment's totals.  With E <= 256 each wave also
//                stores its pairs' IDs as bytes (16 per lane per 1024-pair
//                group) and a flag that says whether the sub-block holds
//                padding or an ID >= E, for the reroute to read instead of
//                the int32 IDs.  The bytes go out as streaming stores, like
//                the reads: cached stores let a reroute that follows soon
//                find part of them in the caches, but cost the histogram
//                itself 10 % and gained the overlapped path under 1 %.
//   scan_kernel  per (plan, 64 experts): inclusive scan of the segment totals
//                in place, which leaves base[j] = pairs of segments < j and
//                base[nseg] = the plan's total; writes load[p][e] and the
//                plan's status word.
// Integer counts only, so the result does not depend on atomic order.
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kHistWaves = kSegSubs;

// the low bytes of four IDs, first ID in the lowest byte
__device__ __forceinline__ uint32_t pack_bytes(i32x4 x) {
    return ((uint32_t)x.x & 0xffu) | (((uint32_t)x.y & 0xffu) << 8) | (((uint32_t)x.z & 0xffu) << 16) |
           ((uint32_t)x.w << 24);
}

__global__ __launch_bounds__(kHistWaves * kWave) void hist_kernel(
    const int32_t *__restrict__ ids, int64_t N, int32_t E, int64_t sub, int64_t nsb,
    int64_t nseg, int32_t *__restrict__ ws, int32_t *__restrict__ flags, uint8_t *__restrict__ ids8,
    int64_t stride8) {
    extern __shared__ int32_t sh_hist[];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int E1 = E + 1;
    int32_t *h = sh_hist + wave * E1;
    const int64_t seg = blockIdx.x;
    const int p = blockIdx.y;
    const int64_t sb = seg * kHistWaves + wave;

    for (int e = lane; e < E1; e += kWave) h[e] = 0;
    wave_lds_fence();

    const int32_t *src = ids + (int64_t)p * N;
    const uint32_t uE = (uint32_t)E;
    int nbad = 0;
    bool odd = false;  // padding or an ID >= E seen
    auto count = [&](int32_t v) {
        if ((uint32_t)v < uE) {
            atomicAdd(&h[v], 1);
        } else {
            odd = true;
            if (v >= E) nbad++;
        }
    };
    uint8_t *row8 = ids8 ? ids8 + (int64_t)p * stride8 : nullptr;

    if (sb < nsb) {  // waves past the plan's last sub-block keep an empty histogram
        const int64_t begin = sb * sub;
        const int64_t end = (begin + sub < N) ? begin + sub : N;
        int64_t i = begin;
        const int64_t ngroup = (end - begin) / kGroupPairs;
        // 16-byte path: the plan row and sub-block start are 16-byte aligned
        if (((uintptr_t)(src + begin) & 15) == 0) {
            const int64_t nvec = (end - begin) / 4;
            const i32x4 *v4 = reinterpret_cast<const i32x4 *>(src + begin);
            constexpr int U = kGroupTiles;
            // whole groups, double-buffered: the next group loads while this
            // one is counted; lane l's IDs of the group go out as 16 bytes
            i32x4 nx[U];
            if (ngroup > 0) {
#pragma unroll
                for (int u = 0; u < U; u++) nx[u] = __builtin_nontemporal_load(v4 + lane + u * kWave);
            }
            for (int64_t gi = 0; gi < ngroup; gi++) {
                i32x4 x[U];
#pragma unroll
                for (int u = 0; u < U; u++) x[u] = nx[u];
                if (gi + 1 < ngroup) {
#pragma unroll
                    for (int u = 0; u < U; u++)
                        nx[u] = __builtin_nontemporal_load(v4 + (gi + 1) * U * kWave + lane + u * kWave);
                }
#pragma unroll
                for (int u = 0; u < U; u++) {
                    count(x[u].x); count(x[u].y); count(x[u].z); count(x[u].w);
                }
                if (row8) {
                    u32x4 b;
                    b.x = pack_bytes(x[0]); b.y = pack_bytes(x[1]); b.z = pack_bytes(x[2]); b.w = pack_bytes(x[3]);
                    __builtin_nontemporal_store(b, reinterpret_cast<u32x4 *>(row8 + begin) + gi * kWave + lane);
                }
            }
            // the rest of the whole vectors; their bytes in pair order
            for (int64_t k = ngroup * U * kWave + lane; k < nvec; k += kWave) {
                const i32x4 x = __builtin_nontemporal_load(v4 + k);
                count(x.x); count(x.y); count(x.z); count(x.w);
                if (row8) __builtin_nontemporal_store(pack_bytes(x), reinterpret_cast<uint32_t *>(row8 + begin) + k);
            }
            i = begin + nvec * 4;
        }
        for (int64_t j = i + lane; j < end; j += kWave) {
            const int32_t v = src[j];
            count(v);
            if (row8) row8[begin + compact_pos(j - begin, ngroup)] = (uint8_t)v;
        }
        if (nbad) atomicAdd(&h[E], nbad);
        if (flags) {
            const bool any = __ballot(odd) != 0;
            if (lane == 0) flags[(int64_t)p * nsb + sb] = any ? 1 : 0;
        }
    }
    __syncthreads();

    int32_t *plan_ws = ws + (int64_t)p * (nsb + nseg + 1) * E1;
    const bool last = wave == kHistWaves - 1;
    if (wave > 0 && (sb < nsb || last)) {
        int32_t *row = plan_ws + sb * E1;
        // segment totals go one row below the segment's base row; the scan
        // makes the rows inclusive in place
        int32_t *tot = plan_ws + (nsb + seg + 1) * E1;
        for (int e = lane; e < E1; e += kWave) {
            int32_t pre = 0;
            for (int w = 0; w < wave; w++) pre += sh_hist[w * E1 + e];
            if (sb < nsb) row[e] = pre;
            if (last) tot[e] = pre + h[e];
        }
    }
    if (kHistWaves == 1) {
        int32_t *tot = plan_ws + (nsb + seg + 1) * E1;
        for (int e = lane; e < E1; e += kWave) tot[e] = h[e];
    }
}

constexpr int kScanUnroll = 8;

template <int kScanWaves>
__global__ __launch_bounds__(kScanWaves * kWave) void scan_kernel(
    int32_t *__restrict__ ws, int64_t nsb, int64_t nseg, int32_t E, int32_t *__restrict__ load,
    uint32_t *__restrict__ status) {
    __shared__ int32_t part[kScanWaves][kWave];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int E1 = E + 1;
    const int p = blockIdx.y;
    const int col = blockIdx.x * kWave + lane;
    // base rows of the plan; rows 1..nseg hold segment totals on entry
    int32_t *base = ws + ((int64_t)p * (nsb + nseg + 1) + nsb) * E1;
    const int64_t per = (nseg + kScanWaves - 1) / kScanWaves;
    const int64_t b0 = 1 + (wave * per < nseg ? wave * per : nseg);
    const int64_t b1 = (b0 + per < nseg + 1) ? b0 + per : nseg + 1;
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
    int32_t run = 0;
    for (int w = 0; w < wave; w++) run += part[w][lane];
    if (on) {
        if (wave == 0) base[col] = 0;
        int64_t b = b0;
        for (; b + kScanUnroll <= b1; b += kScanUnroll) {
            int32_t c[kScanUnroll];
#pragma unroll
            for (int u = 0; u < kScanUnroll; u++) c[u] = base[(b + u) * E1 + col];
#pragma unroll
            for (int u = 0; u < kScanUnroll; u++) {
                run += c[u];
                base[(b + u) * E1 + col] = run;
            }
        }
        for (; b < b1; b++) {
            run += base[b * E1 + col];
            base[b * E1 + col] = run;
        }
        if (wave == kScanWaves - 1) {
            // the last wave's running sum is the plan's total
            if (col < E) load[(int64_t)p * E + col] = run;
            else status[p] = run > 0 ? (uint32_t)EP_STATUS_BAD_ID : 0u;
        }
    }
}

}  // namespace

hipError_t launch_histogram(const int32_t *ids, int64_t N, int32_t P, int32_t E, const SubGeom &g,
                            int32_t *ws, const Compact &cp, int32_t *load, uint32_t *status,
                            hipStream_t s) {
    if (g.sps != kHistWaves) return hipErrorInvalidValue;
    if (g.nseg > 0) {
        dim3 grid((unsigned)g.nseg, (unsigned)P);
        const size_t lds = (size_t)kHistWaves * (E + 1) * sizeof(int32_t);
        hipLaunchKernelGGL(hist_kernel, grid, dim3(kHistWaves * kWave), lds, s, ids, N, E, g.sub,
                           g.nsb, g.nseg, ws, cp.flags, cp.bytes, cp.stride);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // 4-wave workgroups start on CUs busy with other kernels (a concurrent
    // reroute); a launch of a few plans with many segments gets 16 waves per
    // column block, each scanning a quarter of the segments a 4-wave one would
    const unsigned cb = (unsigned)((E + 1 + kWave - 1) / kWave);
    dim3 g2(cb, (unsigned)P);
    if ((int64_t)cb * P <= 16 && g.nseg >= 128)
        hipLaunchKernelGGL(scan_kernel<16>, g2, dim3(16 * kWave), 0, s, ws, g.nsb, g.nseg, E, load, status);
    else
        hipLaunchKernelGGL(scan_kernel<4>, g2, dim3(4 * kWave), 0, s, ws, g.nsb, g.nseg, E, load, status);
    return hipGetLastError();
}

}  // namespace ep
