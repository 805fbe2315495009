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
    // instance rows as codes: h >= 0 the native row of expert h, -1 - o the
    // o-th spare slot's row, kNoRow not a plan's table (codes rather than
    // pointers: a pointer read back from LDS is generic, and its loads would
    // be flat ones, which the LDS wait counter also tracks)
    constexpr int32_t kNoRow = INT32_MIN;
    __shared__ int32_t rows[64];
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
        rows[threadIdx.x] = home >= 0 ? home : (o >= 0 ? -1 - o : kNoRow);
    }
    __syncthreads();
    for (int t = 0; t < c; t++)
        if (rows[t] == kNoRow) return;   // not a plan's table: leave the row alone
    const int64_t c0 = (int64_t)blockIdx.x * kRedChunk;
    const int64_t c1 = (c0 + kRedChunk < vpe) ? c0 + kRedChunk : vpe;
    f32x4 *out = native + (int64_t)e * vpe;
    auto row = [&](int t) -> const f32x4 * {
        const int32_t r = rows[t];
        return r >= 0 ? native + (int64_t)r * vpe : slot + (int64_t)(-1 - r) * vpe;
    };
    // all kRedIters vectors of a thread load together, two rows per step (more
    // loads in flight), non-temporal as every byte is touched once.  The loads
    // are unconditional, from an index clamped to the chunk, so that the wait
    // for one row does not also wait for the other; lanes past the chunk's end
    // fold whatever they read and store nothing.  Each element still folds its
    // rows in slot order, one fp32 add at a time.
    int64_t idx[kRedIters];
#pragma unroll
    for (int k = 0; k < kRedIters; k++) {
        const int64_t i = c0 + threadIdx.x + k * kRedThreads;
        idx[k] = i < c1 ? i : c1 - 1;
    }
    f32x4 acc[kRedIters];
    {
        const f32x4 *r0 = row(0);
#pragma unroll
        for (int k = 0; k < kRedIters; k++) acc[k] = __builtin_nontemporal_load(r0 + idx[k]);
    }
    auto add = [&](f32x4 &a, const f32x4 &g) {
        a.x = a.x + g.x;
        a.y = a.y + g.y;
        a.z = a.z + g.z;
        a.w = a.w + g.w;
    };
    int t = 1;
    for (; t + 1 < c; t += 2) {
        const f32x4 *ra = row(t), *rb = row(t + 1);
        f32x4 ga[kRedIters], gb[kRedIters];
#pragma unroll
        for (int k = 0; k < kRedIters; k++) ga[k] = __builtin_nontemporal_load(ra + idx[k]);
#pragma unroll
        for (int k = 0; k < kRedIters; k++) gb[k] = __builtin_nontemporal_load(rb + idx[k]);
#pragma unroll
        for (int k = 0; k < kRedIters; k++) add(acc[k], ga[k]);
#pragma unroll
        for (int k = 0; k < kRedIters; k++) add(acc[k], gb[k]);
    }
    if (t < c) {
        const f32x4 *ra = row(t);
        f32x4 ga[kRedIters];
#pragma unroll
        for (int k = 0; k < kRedIters; k++) ga[k] = __builtin_nontemporal_load(ra + idx[k]);
#pragma unroll
        for (int k = 0; k < kRedIters; k++) add(acc[k], ga[k]);
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
