// Internal definitions shared by the HIP kernels and the C-ABI entry points.
// gfx950 (CDNA4) only: wave64, LDS atomics, 16-byte global accesses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep_balance.h"

namespace ep {

constexpr int kWave = 64;
// LDS per workgroup on gfx950 (160 KB per CU, all of it addressable by one
// workgroup), and the budget the launchers prefer so that several workgroups
// share a CU; a shape that needs more than the preferred budget runs with
// fewer, larger-LDS workgroups
constexpr size_t kLdsMax = 160 * 1024;
constexpr size_t kLdsPreferred = 64 * 1024;

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Packed layout tables (int32, device), in this order:
//   rank_first [R+1]  first physical slot of each rank (rank-major numbering)
//   rank_nat   [R]    native slots at the start of each rank
//   slot_home  [Phi]  native expert of a slot, -1 for a spare slot
//   slot_rank  [Phi]  rank owning a slot
//   home_slot  [E]    native slot of each expert
//   spare_slot [S]    physical slot of the o-th spare slot (ascending)
//   slot_spare [Phi]  spare ordinal of a slot, -1 for a native slot
// ---------------------------------------------------------------------------
struct Tables {
    const int32_t *rank_first, *rank_nat, *slot_home, *slot_rank, *home_slot, *spare_slot, *slot_spare;
};

inline size_t table_ints(int E, int R, int S) {
    return (size_t)(2 * R + 1) + 3 * (size_t)(E + S) + (size_t)E + (size_t)S;
}

inline Tables tables_of(const ep_layout_t &L) {
    const int R = L.num_ranks, Phi = L.num_phys, E = L.num_experts;
    Tables t;
    t.rank_first = L.tables;
    t.rank_nat = t.rank_first + (R + 1);
    t.slot_home = t.rank_nat + R;
    t.slot_rank = t.slot_home + Phi;
    t.home_slot = t.slot_rank + Phi;
    t.spare_slot = t.home_slot + E;
    t.slot_spare = t.spare_slot + L.num_spare;
    return t;
}

// ---------------------------------------------------------------------------
// Sub-blocks: the pairs of one plan are cut into consecutive sub-blocks, one
// per wave in the reroute and the dispatch layout.  The size aims at ~8K waves
// in a launch (so a launch of one or a few plans gets small sub-blocks and
// more waves), keeps the count table under 1/2 byte per pair with E <= 256
// (>= 8 (E+1) pairs) and under 1/4 byte otherwise (>= 16 (E+1)), and is a
// power of two between 1024 and 4096 unless that bound asks for more.
//
// Segments: the histogram gives each workgroup a segment of `sps`
// consecutive sub-blocks, one per wave.  After counting, each wave stores the
// count of the segment's pairs before its sub-block (the in-segment prefix,
// summed over the lower waves' LDS histograms) and the last wave the
// segment's totals.  A small scan then turns the segment totals into
// exclusive segment bases.  Workspace rows per plan (each E + 1 ints, column
// E counting IDs >= E):
//   rows [0, nsb)              in-segment prefix of sub-block sb (row of a
//                              segment's first sub-block unused: it is 0)
//   rows [nsb, nsb + nseg]     base[j] = pairs of segments < j; base[nseg]
//                              is the plan's total per expert (its load)
// so that the pairs of expert e before sub-block sb number
//   in[sb][e] + base[sb / sps][e].
// ---------------------------------------------------------------------------
#ifndef EP_SUB_TARGET_WAVES
#define EP_SUB_TARGET_WAVES 8192
#endif
#ifndef EP_SUB_MAX
#define EP_SUB_MAX 4096
#endif
#ifndef EP_SUB_MIN
#define EP_SUB_MIN 1024
#endif
#ifndef EP_SEG_SUBS
#define EP_SEG_SUBS 8
#endif
constexpr int kSegSubs = EP_SEG_SUBS;  // sub-blocks per segment = waves per histogram workgroup
inline int64_t sub_pairs(int64_t N, int32_t P, int32_t E) {
    const int64_t tw = EP_SUB_TARGET_WAVES;
    int64_t want = (N * (int64_t)P + tw - 1) / tw;
    // at least 8 (E + 1) pairs when the IDs get a byte copy (E <= 256), else
    // 16 (E + 1): the count table stays under 1/2 or 1/4 byte per pair
    int64_t lo = (E <= 256 ? 8 : 16) * (int64_t)(E + 1);
    if (lo < EP_SUB_MIN) lo = EP_SUB_MIN;
    if (want < lo) want = lo;
    int64_t sub = EP_SUB_MIN;
    while (sub < want && sub < EP_SUB_MAX) sub <<= 1;
    while (sub < lo) sub <<= 1;
#ifdef EP_SUB_FIXED
    sub = EP_SUB_FIXED;
#endif
    return sub;
}

inline int64_t num_sub(int64_t N, int64_t sub) { return N <= 0 ? 0 : (N + sub - 1) / sub; }

// sub-blocks per histogram segment
inline int64_t seg_subs(int64_t, int32_t) { return kSegSubs; }

inline int64_t num_seg(int64_t nsb, int64_t sps) { return (nsb + sps - 1) / sps; }

struct SubGeom {
    int64_t sub, nsb, sps, nseg;
};

inline SubGeom sub_geom(int64_t N, int32_t P, int32_t E) {
    SubGeom g;
    g.sub = sub_pairs(N, P, E);
    g.nsb = num_sub(N, g.sub);
    g.sps = seg_subs(g.nsb, P);
    g.nseg = num_seg(g.nsb, g.sps);
    return g;
}

// ---------------------------------------------------------------------------
// Compact IDs (E <= 256).  Besides counting, the histogram stores every pair's
// ID as one byte and, per sub-block, a flag that is set when the sub-block
// holds padding or an ID >= E.  The reroute of an unflagged sub-block reads
// the bytes instead of the int32 IDs, so the IDs cross HBM as 4 + 1 (written)
// + 1 bytes per pair instead of 4 + 4.  Workspace parts, each 256-byte aligned:
//   count rows  int32 [P][nsb + nseg + 1][E + 1]  (above)
//   flags       int32 [P][nsb]                     (compact only)
//   bytes       uint8 [P][nb], nb = N rounded up to 16 (compact only)
// ---------------------------------------------------------------------------
constexpr int32_t kCompactMaxE = 256;
inline bool compact_ids(int32_t E) { return E <= kCompactMaxE; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline int64_t compact_stride(int64_t N) { return (N + 15) & ~(int64_t)15; }

struct WsParts {
    size_t flags, bytes, total;  // byte offsets of the compact parts (0: none), total size
};

inline WsParts ws_parts(int64_t N, int32_t P, int32_t E) {
    const SubGeom g = sub_geom(N, P, E);
    const size_t rows = (size_t)P * (size_t)(g.nsb + g.nseg + 1) * (size_t)(E + 1) * sizeof(int32_t);
    WsParts w{0, 0, rows};
    if (compact_ids(E) && g.nsb > 0) {
        w.flags = align256(rows);
        w.bytes = w.flags + align256((size_t)P * (size_t)g.nsb * sizeof(int32_t));
        w.total = w.bytes + (size_t)P * (size_t)compact_stride(N);
    }
    return w;
}

inline size_t ws_bytes(int64_t N, int32_t P, int32_t E) { return ws_parts(N, P, E).total; }

// Byte order of the copy within a sub-block.  Whole groups of 1024 pairs (4
// tiles of 256: lane l holds pairs 4l..4l+3 of a tile) are stored lane-major,
// lane l's 16 bytes holding its 4 IDs of each of the 4 tiles, so that one
// 16-byte access per lane moves a group; the pairs after the last whole group
// are stored in order.
constexpr int kGroupTiles = 4;
constexpr int64_t kTilePairs = 4 * kWave;
constexpr int64_t kGroupPairs = kGroupTiles * kTilePairs;

// byte offset of pair j of a sub-block with `ngroup` whole groups
__device__ __forceinline__ int64_t compact_pos(int64_t j, int64_t ngroup) {
    if (j >= ngroup * kGroupPairs) return j;
    const int64_t g = j / kGroupPairs;
    const int r = (int)(j - g * kGroupPairs);
    const int tile = r / (int)kTilePairs, l = (r % (int)kTilePairs) / 4, k = r % 4;
    return g * kGroupPairs + l * 16 + tile * 4 + k;
}

// Device pointers of the compact parts of a workspace (null when E > 256).
struct Compact {
    int32_t *flags;  // [P][nsb]
    uint8_t *bytes;  // [P][stride]
    int64_t stride;
};

inline Compact compact_of(void *ws, int64_t N, int32_t P, int32_t E) {
    const WsParts w = ws_parts(N, P, E);
    Compact c{nullptr, nullptr, compact_stride(N)};
    if (w.flags) {
        c.flags = reinterpret_cast<int32_t *>(static_cast<unsigned char *>(ws) + w.flags);
        c.bytes = static_cast<uint8_t *>(ws) + w.bytes;
    }
    return c;
}

// Per-expert pair counts of plan p before sub-block sb (start) and before
// sb + 1 (end), read from the workspace rows above.
struct SubPrefix {
    const int32_t *in0, *in1, *b0, *b1;
    bool first, last;
    __device__ __forceinline__ int32_t start(int e) const { return (first ? 0 : in0[e]) + b0[e]; }
    __device__ __forceinline__ int32_t end(int e) const { return last ? b1[e] : in1[e] + b0[e]; }
};

__device__ __forceinline__ SubPrefix sub_prefix(const int32_t *ws, int p, int64_t sb, int64_t nsb,
                                                int64_t sps, int64_t nseg, int E1) {
    const int32_t *plan = ws + (int64_t)p * (nsb + nseg + 1) * E1;
    const int64_t seg = sb / sps;
    SubPrefix s;
    s.in0 = plan + sb * E1;
    s.in1 = s.in0 + E1;
    s.b0 = plan + (nsb + seg) * E1;
    s.b1 = s.b0 + E1;
    s.first = sb == seg * sps;
    s.last = sb + 1 == nsb || sb + 1 == (seg + 1) * sps;
    return s;
}

// ---------------------------------------------------------------------------
// wave64 primitives
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() {
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    const uint32_t lo = __shfl_xor((unsigned)(v & 0xffffffffu), m);
    const uint32_t hi = __shfl_xor((unsigned)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ int64_t shfl_up_i64(int64_t v, int d) {
    const uint64_t u = (uint64_t)v;
    const uint32_t lo = __shfl_up((unsigned)(u & 0xffffffffu), d);
    const uint32_t hi = __shfl_up((unsigned)(u >> 32), d);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) {
        const uint64_t o = shfl_xor_u64(v, m);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ int64_t wave_incl_scan_i64(int64_t v) {
    const int l = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int64_t o = shfl_up_i64(v, d);
        if (l >= d) v += o;
    }
    return v;
}

__device__ __forceinline__ int wave_incl_scan_i32(int v) {
    const int l = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(v, d);
        if (l >= d) v += o;
    }
    return v;
}

__device__ __forceinline__ int64_t readlane_i64(int64_t v, int lane) {
    const uint64_t u = (uint64_t)v;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(u & 0xffffffffu), lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(u >> 32), lane);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Wave-wide max / min without LDS: four DPP steps inside each row of 16 lanes
// (quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E, row_half_mirror = 0x141,
// row_mirror = 0x140, fused into the max / min), then gfx950's lane swaps
// across rows (permlane16) and halves (permlane32).  All 64 lanes must be
// active: bound_ctrl reads 0 from a disabled lane.
__device__ __forceinline__ int wave_max_i32(int v) {
    v = max(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true));
    v = max(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true));
    v = max(v, __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true));
    v = max(v, __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true));
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max((int)a[0], (int)a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __builtin_amdgcn_readfirstlane(max((int)b[0], (int)b[1]));
}

__device__ __forceinline__ int wave_min_i32(int v) {
    v = min(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true));
    v = min(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true));
    v = min(v, __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true));
    v = min(v, __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true));
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = min((int)a[0], (int)a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __builtin_amdgcn_readfirstlane(min((int)b[0], (int)b[1]));
}

// orders LDS accesses of the lanes of one wave (no workgroup barrier)
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Workgroups of kernel `fn` (threads per workgroup, dynamic LDS bytes) that
// the current device holds at once, 0 if unknown.  Cached per (device, fn,
// threads, lds), so launches make no runtime queries after the first.
int resident_blocks(const void *fn, int threads, size_t lds);

// ---------------------------------------------------------------------------
// launchers (defined in the .hip files; return hipError_t of the launch)
// ---------------------------------------------------------------------------
// Host-side argument checks of ep_load_histogram, ep_plan_quota and
// ep_reroute (EP_OK or the error code the call returns); the no-allocation
// chain runs all three before it enqueues anything.
int check_histogram(const int32_t *topk_ids, int64_t N, int32_t P, const ep_layout_t *layout,
                    const int32_t *load, const void *ws, size_t ws_size, const uint32_t *status);
int check_plan(const int32_t *load, int32_t P, const ep_layout_t *layout, const int32_t *phy2log,
               const int32_t *phy_quota, const int32_t *logcnt, const int32_t *log2phy);
int check_reroute(const int32_t *topk_ids, int64_t N, int32_t P, const ep_layout_t *layout,
                  const int32_t *phy_quota, const int32_t *log2phy, const int32_t *logcnt, const void *ws,
                  size_t ws_size, const int32_t *phys_ids);

hipError_t launch_histogram(const int32_t *ids, int64_t N, int32_t P, int32_t E, const SubGeom &g,
                            int32_t *ws, const Compact &cp, int32_t *load, uint32_t *status,
                            hipStream_t s);
// cfg > 0 selects the rank-per-lane planner (32 * natives + spares registers
// per lane, see plan_lanes_cfg); cfg == 0 selects the generic planner
hipError_t launch_plan(const int32_t *load, int32_t P, const ep_layout_t &L, int32_t *phy2log,
                       int32_t *phy_quota, int32_t *logcnt, int32_t *log2phy, int32_t *steps,
                       uint32_t *status, hipStream_t s, int cfg);
size_t plan_lds_bytes(const ep_layout_t &L);
int plan_lanes_cfg(const ep_layout_t &L);
hipError_t launch_reroute(const int32_t *ids, int64_t N, int32_t P, const ep_layout_t &L,
                          const SubGeom &g, const int32_t *ws, const Compact &cp,
                          const int32_t *phy_quota, const int32_t *log2phy, const int32_t *logcnt,
                          int32_t *out, hipStream_t s);
size_t reroute_lds_bytes(int E, int Phi, int waves);
hipError_t launch_dispatch(const int32_t *ids, int64_t N, int32_t P, const ep_layout_t &L,
                           const SubGeom &g, const int32_t *ws, const int32_t *phy_quota,
                           const int32_t *log2phy, const int32_t *logcnt, int32_t *slot_offsets,
                           int32_t *dpos, int32_t *dsrc, hipStream_t s);
size_t dispatch_lds_bytes(int E, int Phi, int waves, int64_t stage_pairs, bool pair);
hipError_t launch_grad_reduce(float *native, int64_t n, const float *slot, const int32_t *log2phy,
                              const int32_t *logcnt, const ep_layout_t &L, hipStream_t s);
// ws: the fill-list workspace (fill_ws_bytes(S) bytes) or null
hipError_t launch_slot_fill(const void *w, int64_t bytes_per_expert, const int32_t *phy2log,
                            const ep_layout_t &L, void *buf, int32_t *ws, hipStream_t s);
size_t fill_ws_bytes(int32_t S);
hipError_t launch_stats(const int32_t *load, const int32_t *phy_quota, int32_t P,
                        const ep_layout_t &L, int64_t *stats, double *imbalance,
                        int32_t *rank_load, hipStream_t s);

}  // namespace ep
