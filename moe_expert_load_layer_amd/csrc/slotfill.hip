// A4: weight distribution on one GPU (UltraEP news article, section on the key
// designs: replicas live in slots reserved per rank, and one slot buffer is
// reused by every layer).  For the o-th spare slot s with phy2log[s] = e >= 0,
// expert e's weights are copied into row o of the slot buffer; empty slots are
// not written.  A pure HBM-to-HBM stream of 16-byte loads and stores, each
// workgroup of 256 threads moving one 16 KiB chunk.
//
// A hot expert often has several replicas, in different slots of one plan.
// The chunk of such an expert is read once, by the workgroup of its lowest
// spare slot, and stored into every slot that holds it (the other slots'
// workgroups return at once), so the stream moves (distinct experts + used
// slots) x bytes_per_expert instead of 2 x used slots.  Workgroups are
// numbered chunk-major, each chunk's slots rotated by the chunk index: the
// workgroups resident at one time copy the same chunk of many slots (many
// distant streams) and every slot's chunks spread over all XCDs (the
// hardware hands consecutive workgroups to the 8 XCDs in turn), so empty
// slots leave no XCD idle.  Up to kDedupMaxSpare spare slots; beyond that,
// slot-major order without sharing.
#include "ep_internal.h"

namespace ep {
namespace {

#ifndef EP_FILL_THREADS
#define EP_FILL_THREADS 256
#endif
#ifndef EP_FILL_UNROLL
#define EP_FILL_UNROLL 4
#endif
#ifndef EP_FILL_CHUNK_ITERS
#define EP_FILL_CHUNK_ITERS 1
#endif
#ifndef EP_FILL_SHARED
#define EP_FILL_SHARED 1
#endif
constexpr int kFillThreads = EP_FILL_THREADS;
constexpr int kFillUnroll = EP_FILL_UNROLL;
constexpr int64_t kFillChunk = (int64_t)kFillThreads * kFillUnroll * EP_FILL_CHUNK_ITERS;  // 16-byte vectors

// Weights are loaded through the caches; slot rows are stored as streaming
// (nontemporal) writes: nothing in this launch reads them back, and keeping them
// out of L2 measured 1 to 2% faster per layer on every workload.
#define LD(p) (*(p))
#define ST(v, p) __builtin_nontemporal_store(v, p)

__global__ __launch_bounds__(kFillThreads) void slot_fill_kernel(
    const u32x4 *__restrict__ w, int64_t vpe, int32_t E, const int32_t *__restrict__ phy2log,
    const int32_t *__restrict__ spare_slot, u32x4 *__restrict__ buf) {
    const int o = blockIdx.y;
    const int e = phy2log[spare_slot[o]];
    if (e < 0 || e >= E) return;
    const int64_t c0 = (int64_t)blockIdx.x * kFillChunk;
    const int64_t c1 = (c0 + kFillChunk < vpe) ? c0 + kFillChunk : vpe;
    const u32x4 *src = w + (int64_t)e * vpe;
    u32x4 *dst = buf + (int64_t)o * vpe;
    int64_t i = c0 + threadIdx.x;
    for (; i + (kFillUnroll - 1) * kFillThreads < c1; i += kFillUnroll * kFillThreads) {
        u32x4 x[kFillUnroll];
#pragma unroll
        for (int u = 0; u < kFillUnroll; u++) x[u] = LD(src + i + u * kFillThreads);
#pragma unroll
        for (int u = 0; u < kFillUnroll; u++) ST(x[u], dst + i + u * kFillThreads);
    }
    for (; i < c1; i += kFillThreads) ST(LD(src + i), dst + i);
}

constexpr int kDedupMaxSpare = 1024;
static_assert(EP_FILL_CHUNK_ITERS == 1, "a shared-fill workgroup holds its whole chunk in registers");

__global__ __launch_bounds__(kFillThreads) void slot_fill_shared_kernel(
    const u32x4 *__restrict__ w, int64_t vpe, int32_t E, const int32_t *__restrict__ phy2log,
    const int32_t *__restrict__ spare_slot, int32_t S, u32x4 *__restrict__ buf) {
    const int64_t nb = gridDim.x;  // chunks per slot
    const int64_t L = (int64_t)blockIdx.y * nb + blockIdx.x;
    const int64_t cb = L / S;
    const int o = (int)((L % S + cb) % S);
    const int e = phy2log[spare_slot[o]];
    if (e < 0 || e >= E) return;
    const int lane = threadIdx.x % kWave;
    // the lowest spare slot holding e does the work
    for (int base = 0; base < o; base += kWave) {
        const int j = base + lane;
        const bool hit = j < o && phy2log[spare_slot[j]] == e;
        if (__ballot(hit)) return;  // the same answer in every wave
    }
    const int64_t c0 = cb * kFillChunk;
    const int64_t c1 = (c0 + kFillChunk < vpe) ? c0 + kFillChunk : vpe;
    const u32x4 *src = w + (int64_t)e * vpe;
    const int64_t i0 = c0 + threadIdx.x;
    u32x4 x[kFillUnroll];
#pragma unroll
    for (int u = 0; u < kFillUnroll; u++) {
        const int64_t i = i0 + u * kFillThreads;
        if (i < c1) x[u] = LD(src + i);
    }
    // store into every slot holding e, from o on (the slot list is read while
    // the chunk loads)
    for (int base = o; base < S; base += kWave) {
        const int j = base + lane;
        for (uint64_t m = __ballot(j < S && phy2log[spare_slot[j]] == e); m; m &= m - 1) {
            u32x4 *dst = buf + (int64_t)(base + __ffsll((long long)m) - 1) * vpe;
#pragma unroll
            for (int u = 0; u < kFillUnroll; u++) {
                const int64_t i = i0 + u * kFillThreads;
                if (i < c1) ST(x[u], dst + i);
            }
        }
    }
}

}  // namespace

hipError_t launch_slot_fill(const void *w, int64_t bytes_per_expert, const int32_t *phy2log,
                            const ep_layout_t &L, void *buf, hipStream_t s) {
    if (L.num_spare == 0) return hipSuccess;
    const int64_t vpe = bytes_per_expert / 16;
    dim3 grid((unsigned)((vpe + kFillChunk - 1) / kFillChunk), (unsigned)L.num_spare);
    if (L.num_spare <= kDedupMaxSpare && EP_FILL_SHARED) {
        hipLaunchKernelGGL(slot_fill_shared_kernel, grid, dim3(kFillThreads), 0, s,
                           reinterpret_cast<const u32x4 *>(w), vpe, L.num_experts, phy2log,
                           tables_of(L).spare_slot, L.num_spare, reinterpret_cast<u32x4 *>(buf));
    } else {
        hipLaunchKernelGGL(slot_fill_kernel, grid, dim3(kFillThreads), 0, s,
                           reinterpret_cast<const u32x4 *>(w), vpe, L.num_experts, phy2log,
                           tables_of(L).spare_slot, reinterpret_cast<u32x4 *>(buf));
    }
    return hipGetLastError();
}

}  // namespace ep
