// Replica gradient reduction in backward (UltraEP article, key designs:
// replica gradients are reduced back to the native expert; backward
// paragraph: accumulation keeps a fixed order so it is deterministic).
//
// Grid: (16 KiB chunks of one expert's gradient, experts).  A workgroup of an
// expert with fewer than two instances exits at once.  Otherwise the first
// wave resolves the expert's instance rows (ascending physical slot: the
// native row or the replica's spare-slot row) into LDS, and every thread
// folds its 4 floats over the rows in that order, one fp32 add at a time,
// then overwrites the native row.  Pure HBM streaming: (instances + 1) rows
// of n floats per replicated expert.
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kRedThreads = 256;
constexpr int kRedIters = 4;
constexpr int64_t kRedChunk = (int64_t)kRedThreads * kRedIters;  // float4 vectors

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kRedThreads) void grad_reduce_kernel(
    f32x4 *__restrict__ native, int64_t vpe, const f32x4 *__restrict__ slot,
    const int32_t *__restrict__ log2phy, const int32_t *__restrict__ logcnt, int32_t rho,
    int32_t Phi, Tables T) {
    __shared__ const f32x4 *rows[64];
    const int e = blockIdx.y;
    int c = logcnt[e];
    c = c > rho ? rho : c;
    c = c > 64 ? 64 : c;  // the entry point admits rho <= 64 only
    if (c < 2) return;
    if (threadIdx.x < c) {
        const int s = log2phy[(int64_t)e * rho + threadIdx.x];
        const bool ok = s >= 0 && s < Phi;
        const int home = ok ? T.slot_home[s] : -1;
        const int o = ok ? T.slot_spare[s] : -1;
        rows[threadIdx.x] = home >= 0 ? native + (int64_t)home * vpe
                                      : (o >= 0 ? slot + (int64_t)o * vpe : nullptr);
    }
    __syncthreads();
    for (int t = 0; t < c; t++)
        if (rows[t] == nullptr) return;   // not a plan's table: leave the row alone
    const int64_t c0 = (int64_t)blockIdx.x * kRedChunk;
    const int64_t c1 = (c0 + kRedChunk < vpe) ? c0 + kRedChunk : vpe;
    f32x4 *out = native + (int64_t)e * vpe;
    // all kRedIters vectors of a thread load together for each row (more
    // loads in flight), non-temporal as every byte is touched once; each
    // element still folds its rows in slot order
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc[kRedIters];
#pragma unroll
    for (int k = 0; k < kRedIters; k++) {
        const int64_t i = c0 + threadIdx.x + k * kRedThreads;
        acc[k] = i < c1 ? __builtin_nontemporal_load(rows[0] + i) : zero;
    }
    for (int t = 1; t < c; t++) {
        f32x4 g[kRedIters];
#pragma unroll
        for (int k = 0; k < kRedIters; k++) {
            const int64_t i = c0 + threadIdx.x + k * kRedThreads;
            g[k] = i < c1 ? __builtin_nontemporal_load(rows[t] + i) : zero;
        }
#pragma unroll
        for (int k = 0; k < kRedIters; k++) {
            acc[k].x = acc[k].x + g[k].x;
            acc[k].y = acc[k].y + g[k].y;
            acc[k].z = acc[k].z + g[k].z;
            acc[k].w = acc[k].w + g[k].w;
        }
    }
#pragma unroll
    for (int k = 0; k < kRedIters; k++) {
        const int64_t i = c0 + threadIdx.x + k * kRedThreads;
        if (i < c1) __builtin_nontemporal_store(acc[k], out + i);
    }
}

}  // namespace

hipError_t launch_grad_reduce(float *native, int64_t n, const float *slot, const int32_t *log2phy,
                              const int32_t *logcnt, const ep_layout_t &L, hipStream_t s) {
    const int64_t vpe = n / 4;
    dim3 grid((unsigned)((vpe + kRedChunk - 1) / kRedChunk), (unsigned)L.num_experts);
    hipLaunchKernelGGL(grad_reduce_kernel, grid, dim3(kRedThreads), 0, s,
                       reinterpret_cast<f32x4 *>(native), vpe, reinterpret_cast<const f32x4 *>(slot),
                       log2phy, logcnt, L.max_replicas, L.num_phys, tables_of(L));
    return hipGetLastError();
}

}  // namespace ep
