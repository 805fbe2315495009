// A4: weight distribution on one GPU (UltraEP news article, section on the key
// designs: replicas live in slots reserved per rank, and one slot buffer is
// reused by every layer).  For the o-th spare slot s with phy2log[s] = e >= 0,
// expert e's weights are copied into row o of the slot buffer; empty slots are
// not written.  A pure HBM-to-HBM stream of 16-byte loads and stores.
//
// A hot expert often has several replicas in one plan.  Each distinct expert
// is read once per item (up to kItemSlots of its slots) and stored into every
// slot of the item, so the stream moves about (distinct experts + filled slots)
// x bytes_per_expert instead of 2 x filled slots.
//
// With a workspace (up to kListMaxSpare spare slots) the fill runs in two
// launches:
//   fill_list_kernel  one workgroup: the plan's fill list, i.e. the distinct
//                     experts among the spare slots in order of their lowest
//                     slot, each cut into items of at most kItemSlots slots, and
//                     for each item the ordinals of its slots, in ascending order;
//   fill_copy_kernel  4 KiB per workgroup (one 16-byte vector per thread),
//                     each chunk of an item read once and stored into every
//                     slot of the item; the workgroups of one item stream
//                     128 KiB of its weights in address order before the next
//                     item's run (see the kernel for the numbering).
// Small workgroups that each move one 16-byte vector per thread keep the most
// bytes in flight; reading an item's rows in address order lets the memory
// stream them.  Without a workspace, or with more spare slots, each workgroup
// finds its slot's expert and the other holders itself
// (slot_fill_shared_kernel, 16 KiB chunks), or above kDedupMaxSpare spare slots
// copies its own slot (slot_fill_kernel).
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kFillThreads = 256;
constexpr int kFillUnroll = 4;
constexpr int64_t kFillChunk = (int64_t)kFillThreads * kFillUnroll;  // 16-byte vectors
constexpr int kListMaxSpare = 1024;
constexpr int kDedupMaxSpare = 1024;
constexpr uint32_t kSuperChunks = 32;  // 4 KiB chunks an item streams before the next item
// Slots per item: an expert held by more spare slots is read once per item of
// at most this many slots, so no workgroup stores one chunk into more than 4
// rows.  Long store fans kept workgroups alive for many serial stores (the
// stress plans hold a hot expert in 20+ slots); per layer, 1 item per expert ->
// at most 4 slots per item: stress 1131 -> 1015 us, Qwen3-like 588 -> 574 us,
// GLM-4.5-like 465 -> 450 us, DeepSeek-V3-like unchanged (2, 3, 5, 6, 8 measured:
// 4 is best or within 1 % everywhere).
constexpr int kItemSlots = 4;

// Weights are loaded through the caches; slot rows are stored as streaming
// (nontemporal) writes: nothing in this launch reads them back.
#define LD(p) (*(p))
#define ST(v, p) __builtin_nontemporal_store(v, p)

// ----------------------------------------------------------------- fill list
// ws layout (int32), n = number of items:
//   [0]                  n
//   [1, 1 + S)           the item's expert, items in order of their first slot
//   [1 + S, 2 + S + n)   the item's first target (and the total after the last)
//   [2 + 2S, 2 + 3S)     the targets: spare ordinals grouped by item, ascending
// A copy workgroup reads n, its item's expert and its two target bounds
// (scalar loads; the words are shared by many workgroups).
__global__ __launch_bounds__(kListMaxSpare) void fill_list_kernel(const int32_t *__restrict__ phy2log,
                                                                 const int32_t *__restrict__ spare_slot,
                                                                 int32_t S, int32_t E,
                                                                 int32_t *__restrict__ ws) {
    __shared__ int32_t key[kListMaxSpare];
    __shared__ int32_t first[kListMaxSpare];  // first target of a leader's item
    __shared__ int32_t scan[kListMaxSpare];
    const int o = threadIdx.x;
    int e = -1;
    if (o < S) {
        e = phy2log[spare_slot[o]];
        if (e < 0 || e >= E) e = -1;
        key[o] = e;
    }
    __syncthreads();
    // The slots holding one expert, in ordinal order, form items of at most
    // kItemSlots slots.  For this ordinal: r = its rank among the expert's
    // holders, lead = the ordinal of its item's first slot, rank = its place in
    // the item, holders = the item's size.
    int lead = o, rank = 0, holders = 0;
    if (o < S && e >= 0) {
        int r = 0, all = 0;
        for (int i = 0; i < S; i++) {
            const bool same = key[i] == e;
            r += (same && i < o) ? 1 : 0;
            all += same ? 1 : 0;
        }
        const int r0 = r - r % kItemSlots;
        lead = -1;
        for (int i = 0, c = 0; i < S; i++) {
            const bool same = key[i] == e;
            if (same && c == r0 && lead < 0) lead = i;
            c += same ? 1 : 0;
        }
        rank = r - r0;
        holders = all - r0 < kItemSlots ? all - r0 : kItemSlots;
    }
    const bool is_lead = o < S && e >= 0 && lead == o;
    // inclusive scan over the leaders (item count in the high half) and their
    // holder counts (targets in the low half), in ordinal order
    const int mine = is_lead ? (1 << 16) | holders : 0;  // counts < 2^16 (S <= 1024)
    scan[o] = mine;
    __syncthreads();
    for (int d = 1; d < kListMaxSpare; d <<= 1) {
        const int v = o >= d ? scan[o - d] : 0;
        __syncthreads();
        scan[o] += v;
        __syncthreads();
    }
    if (is_lead) {
        const int excl = scan[o] - mine;
        first[o] = excl & 0xffff;
        ws[1 + (excl >> 16)] = e;
        ws[1 + S + (excl >> 16)] = excl & 0xffff;
    }
    if (o == kListMaxSpare - 1) {
        const int total = scan[o];
        ws[0] = total >> 16;
        ws[1 + S + (total >> 16)] = total & 0xffff;
    }
    __syncthreads();
    if (o < S && e >= 0) ws[2 + 2 * S + first[lead] + rank] = o;
}

// Workgroup b copies chunk c of item i: in super-chunks of M chunks
// (M = min(kSuperChunks, chunks per expert)), item-major inside each,
// b -> (super-chunk, item, chunk).  An item's workgroups thus stream M
// consecutive chunks (up to 128 KiB) of its expert before the next item's run
// starts, and the workgroups of item numbers past the plan's last item (which
// return at once) are spread over the whole launch instead of all dispatched
// at its end.
__global__ __launch_bounds__(kFillThreads) void fill_copy_kernel(const u32x4 *__restrict__ w, int64_t vpe,
                                                                int64_t nch, int32_t S, uint32_t M,
                                                                const int32_t *__restrict__ ws,
                                                                u32x4 *__restrict__ buf) {
    // (the grid has fewer than 2^31 workgroups: 32-bit index arithmetic)
    const uint32_t b = blockIdx.x;
    const uint32_t per = (uint32_t)S * M;
    const uint32_t sc = b / per, r = b - sc * per;
    const int item = (int)(r / M);
    const int64_t c = (int64_t)sc * M + (r - (uint32_t)item * M);
    if (item >= ws[0] || c >= nch) return;
    const int e = ws[1 + item];
    const int t0 = ws[1 + S + item], t1 = ws[2 + S + item];
    const int32_t *tg = ws + 2 + 2 * S;
    const int64_t i = c * kFillThreads + threadIdx.x;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (i < vpe) x = LD(w + (int64_t)e * vpe + i);
    for (int t = t0; t < t1; t++)
        if (i < vpe) ST(x, buf + (int64_t)tg[t] * vpe + i);
}

// ------------------------------------------------ without a fill list
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

// Workgroups are numbered chunk-major, each chunk's slots rotated by the chunk
// index, so the slots' chunks spread over all XCDs; the workgroup of the
// lowest slot holding an expert loads the chunk and stores it into every slot
// that holds the expert, the others return after that check.
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

size_t fill_ws_bytes(int32_t S) {
    return S <= 0 || S > kListMaxSpare ? 0 : (3 * (size_t)S + 2) * sizeof(int32_t);
}

hipError_t launch_slot_fill(const void *w, int64_t bytes_per_expert, const int32_t *phy2log,
                            const ep_layout_t &L, void *buf, int32_t *ws, hipStream_t s) {
    const int S = L.num_spare;
    if (S == 0) return hipSuccess;
    const int64_t vpe = bytes_per_expert / 16;
    const int64_t nch = (vpe + kFillThreads - 1) / kFillThreads;
    const uint32_t M = nch < (int64_t)kSuperChunks ? (uint32_t)nch : kSuperChunks;
    const int64_t ncopy = (nch + M - 1) / M * M * S;
    if (ws && S <= kListMaxSpare && ncopy <= 0x7fffffffLL) {
        hipLaunchKernelGGL(fill_list_kernel, dim3(1), dim3(kListMaxSpare), 0, s, phy2log,
                           tables_of(L).spare_slot, S, L.num_experts, ws);
        hipLaunchKernelGGL(fill_copy_kernel, dim3((unsigned)ncopy), dim3(kFillThreads), 0, s,
                           reinterpret_cast<const u32x4 *>(w), vpe, nch, S, M, ws,
                           reinterpret_cast<u32x4 *>(buf));
        return hipGetLastError();
    }
    dim3 grid((unsigned)((vpe + kFillChunk - 1) / kFillChunk), (unsigned)S);
    if (S <= kDedupMaxSpare) {
        hipLaunchKernelGGL(slot_fill_shared_kernel, grid, dim3(kFillThreads), 0, s,
                           reinterpret_cast<const u32x4 *>(w), vpe, L.num_experts, phy2log,
                           tables_of(L).spare_slot, S, reinterpret_cast<u32x4 *>(buf));
    } else {
        hipLaunchKernelGGL(slot_fill_kernel, grid, dim3(kFillThreads), 0, s,
                           reinterpret_cast<const u32x4 *>(w), vpe, L.num_experts, phy2log,
                           tables_of(L).spare_slot, reinterpret_cast<u32x4 *>(buf));
    }
    return hipGetLastError();
}

}  // namespace ep
