// C-ABI entry points: argument checks on the host, then kernel launches on the
// caller's stream.  No allocation, no synchronisation (except the one-time
// blocking copy in ep_layout_init).
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "ep_internal.h"

using namespace ep;

namespace {

constexpr size_t kMaxLds = kLdsMax;
constexpr int64_t kMaxPairs = 0x7fffffffLL;
constexpr int32_t kMaxPlans = 65535;

inline hipStream_t as_stream(ep_stream_t s) { return reinterpret_cast<hipStream_t>(s); }
inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline int hip_rc(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ERR_HIP; }

bool layout_ok(const ep_layout_t *L) {
    if (!L || !L->tables) return false;
    if (L->num_experts < 1 || L->num_experts > EP_MAX_EXPERTS) return false;
    if (L->num_ranks < 1 || L->num_ranks > EP_MAX_RANKS) return false;
    if (L->num_spare < 0 || L->num_phys != L->num_experts + L->num_spare) return false;
    const int32_t rho = L->num_ranks < 1 + L->num_spare ? L->num_ranks : 1 + L->num_spare;
    if (L->max_replicas != rho) return false;
    if (L->max_rank_natives < 0 || L->max_rank_natives > L->num_experts) return false;
    if (L->max_rank_spares < 0 || L->max_rank_spares > L->num_spare) return false;
    if (L->ranks_per_domain < 0) return false;
    return aligned(L->tables, 4);
}

bool pairs_ok(const int32_t *ids, int64_t N, int32_t P) {
    if (N < 0 || N > kMaxPairs || P < 1 || P > kMaxPlans) return false;
    if (N > 0 && (!ids || !aligned(ids, 4))) return false;
    return true;
}

}  // namespace

namespace ep {

int check_histogram(const int32_t *topk_ids, int64_t N, int32_t P, const ep_layout_t *layout,
                    const int32_t *load, const void *ws, size_t ws_size, const uint32_t *status) {
    if (!layout_ok(layout) || !pairs_ok(topk_ids, N, P) || !load || !status) return EP_ERR_INVALID_ARG;
    const int E = layout->num_experts;
    if ((size_t)kSegSubs * (E + 1) * 4 > kMaxLds) return EP_ERR_INVALID_ARG;
    const size_t need = ws_bytes(N, P, E);
    if (ws_size < need || (need > 0 && (!ws || !aligned(ws, 16)))) return EP_ERR_INVALID_ARG;
    return EP_OK;
}

int check_plan(const int32_t *load, int32_t P, const ep_layout_t *layout, const int32_t *phy2log,
               const int32_t *phy_quota, const int32_t *logcnt, const int32_t *log2phy) {
    if (!layout_ok(layout) || !load || !phy2log || !phy_quota || !logcnt || !log2phy)
        return EP_ERR_INVALID_ARG;
    if (P < 1 || P > kMaxPlans || layout->max_replicas > 64) return EP_ERR_INVALID_ARG;
    if (plan_lanes_cfg(*layout) == 0 && plan_lds_bytes(*layout) > kMaxLds) return EP_ERR_INVALID_ARG;
    return EP_OK;
}

int check_reroute(const int32_t *topk_ids, int64_t N, int32_t P, const ep_layout_t *layout,
                  const int32_t *phy_quota, const int32_t *log2phy, const int32_t *logcnt, const void *ws,
                  size_t ws_size, const int32_t *phys_ids) {
    if (!layout_ok(layout) || !pairs_ok(topk_ids, N, P) || !phy_quota || !log2phy || !logcnt)
        return EP_ERR_INVALID_ARG;
    if (N > 0 && (!phys_ids || !aligned(phys_ids, 4))) return EP_ERR_INVALID_ARG;
    const int E = layout->num_experts;
    if (reroute_lds_bytes(E, layout->num_phys, 1) > kMaxLds) return EP_ERR_INVALID_ARG;
    const size_t need = ws_bytes(N, P, E);
    if (ws_size < need || (need > 0 && (!ws || !aligned(ws, 16)))) return EP_ERR_INVALID_ARG;
    return EP_OK;
}

}  // namespace ep

extern "C" {

size_t ep_layout_table_ints(int32_t num_experts, int32_t num_ranks, int32_t num_spare) {
    if (num_experts < 1 || num_ranks < 1 || num_spare < 0) return 0;
    return table_ints(num_experts, num_ranks, num_spare);
}

int ep_layout_init(int32_t E, int32_t R, const int32_t *native_count, const int32_t *native_experts,
                   const int32_t *spare_count, int32_t *device_tables, size_t device_table_ints,
                   ep_layout_t *out) {
    if (!native_count || !native_experts || !spare_count || !device_tables || !out)
        return EP_ERR_INVALID_ARG;
    if (E < 1 || E > EP_MAX_EXPERTS || R < 1 || R > EP_MAX_RANKS || !aligned(device_tables, 4))
        return EP_ERR_INVALID_ARG;
    int64_t nat_total = 0, S = 0;
    int32_t max_nat = 0, max_sp = 0;
    for (int r = 0; r < R; r++) {
        if (native_count[r] < 0 || spare_count[r] < 0) return EP_ERR_INVALID_ARG;
        nat_total += native_count[r];
        S += spare_count[r];
        max_nat = native_count[r] > max_nat ? native_count[r] : max_nat;
        max_sp = spare_count[r] > max_sp ? spare_count[r] : max_sp;
    }
    if (nat_total != E || S > (int64_t)EP_MAX_EXPERTS * 64) return EP_ERR_INVALID_ARG;
    const int Phi = E + (int)S;
    const size_t need = table_ints(E, R, (int)S);
    if (device_table_ints < need) return EP_ERR_INVALID_ARG;

    std::vector<int32_t> t(need);
    int32_t *rank_first = t.data();
    int32_t *rank_nat = rank_first + R + 1;
    int32_t *slot_home = rank_nat + R;
    int32_t *slot_rank = slot_home + Phi;
    int32_t *home_slot = slot_rank + Phi;
    int32_t *spare_slot = home_slot + E;
    int32_t *slot_spare = spare_slot + S;
    for (int e = 0; e < E; e++) home_slot[e] = -1;
    int slot = 0, in = 0, o = 0;
    std::vector<int32_t> blk;
    for (int r = 0; r < R; r++) {
        rank_first[r] = slot;
        rank_nat[r] = native_count[r];
        blk.assign(native_experts + in, native_experts + in + native_count[r]);
        in += native_count[r];
        std::sort(blk.begin(), blk.end());  // natives of a rank in ascending logical ID
        for (int32_t e : blk) {
            if (e < 0 || e >= E || home_slot[e] != -1) return EP_ERR_INVALID_ARG;
            home_slot[e] = slot;
            slot_home[slot] = e;
            slot_rank[slot] = r;
            slot_spare[slot] = -1;
            slot++;
        }
        for (int i = 0; i < spare_count[r]; i++) {
            slot_home[slot] = -1;
            slot_rank[slot] = r;
            slot_spare[slot] = o;
            spare_slot[o++] = slot;
            slot++;
        }
    }
    rank_first[R] = slot;
    if (hipMemcpy(device_tables, t.data(), need * sizeof(int32_t), hipMemcpyHostToDevice) != hipSuccess)
        return EP_ERR_HIP;
    out->num_experts = E;
    out->num_ranks = R;
    out->num_phys = Phi;
    out->num_spare = (int32_t)S;
    out->max_replicas = R < 1 + (int32_t)S ? R : 1 + (int32_t)S;
    out->max_rank_natives = max_nat;
    out->max_rank_spares = max_sp;
    out->ranks_per_domain = 0;
    out->tables = device_tables;
    return EP_OK;
}

size_t ep_workspace_bytes(int64_t pairs_per_plan, int32_t num_plans, int32_t num_experts) {
    if (pairs_per_plan < 0 || num_plans < 1 || num_experts < 1) return 0;
    return ws_bytes(pairs_per_plan, num_plans, num_experts);
}

int64_t ep_sub_block_pairs(int64_t pairs_per_plan, int32_t num_plans, int32_t num_experts) {
    if (pairs_per_plan < 0 || num_plans < 1 || num_experts < 1) return 0;
    return sub_pairs(pairs_per_plan, num_plans, num_experts);
}

int ep_load_histogram(const int32_t *topk_ids, int64_t N, int32_t P, const ep_layout_t *layout,
                      int32_t *load, void *ws, size_t ws_size, uint32_t *status,
                      ep_stream_t stream) {
    const int rc = check_histogram(topk_ids, N, P, layout, load, ws, ws_size, status);
    if (rc != EP_OK) return rc;
    const int E = layout->num_experts;
    return hip_rc(launch_histogram(topk_ids, N, P, E, sub_geom(N, P, E), static_cast<int32_t *>(ws),
                                   compact_of(ws, N, P, E), load, status, as_stream(stream)));
}

int ep_plan_quota(const int32_t *load, int32_t P, const ep_layout_t *layout, int32_t *phy2log,
                  int32_t *phy_quota, int32_t *logcnt, int32_t *log2phy, int32_t *steps,
                  uint32_t *status, ep_stream_t stream) {
    const int rc = check_plan(load, P, layout, phy2log, phy_quota, logcnt, log2phy);
    if (rc != EP_OK) return rc;
    const int cfg = plan_lanes_cfg(*layout);
    return hip_rc(launch_plan(load, P, *layout, phy2log, phy_quota, logcnt, log2phy, steps, status,
                              as_stream(stream), cfg));
}

int ep_reroute(const int32_t *topk_ids, int64_t N, int32_t P, const ep_layout_t *layout,
               const int32_t *phy_quota, const int32_t *log2phy, const int32_t *logcnt,
               const void *ws, size_t ws_size, int32_t *phys_ids, ep_stream_t stream) {
    const int rc = check_reroute(topk_ids, N, P, layout, phy_quota, log2phy, logcnt, ws, ws_size, phys_ids);
    if (rc != EP_OK) return rc;
    const int E = layout->num_experts;
    return hip_rc(launch_reroute(topk_ids, N, P, *layout, sub_geom(N, P, E), static_cast<const int32_t *>(ws),
                                 compact_of(const_cast<void *>(ws), N, P, E), phy_quota, log2phy,
                                 logcnt, phys_ids, as_stream(stream)));
}

int ep_dispatch_layout(const int32_t *topk_ids, int64_t N, int32_t P, const ep_layout_t *layout,
                       const int32_t *phy_quota, const int32_t *log2phy, const int32_t *logcnt,
                       const void *ws, size_t ws_size, int32_t *slot_offsets, int32_t *dispatch_pos,
                       int32_t *dispatch_src, ep_stream_t stream) {
    if (!layout_ok(layout) || !pairs_ok(topk_ids, N, P) || !phy_quota || !log2phy || !logcnt ||
        !slot_offsets)
        return EP_ERR_INVALID_ARG;
    if (!aligned(slot_offsets, 4)) return EP_ERR_INVALID_ARG;
    if (N > 0 && (!dispatch_pos || !dispatch_src || !aligned(dispatch_pos, 4) || !aligned(dispatch_src, 4)))
        return EP_ERR_INVALID_ARG;
    const int E = layout->num_experts;
    if (dispatch_lds_bytes(E, layout->num_phys, 1, 0, false) > kMaxLds) return EP_ERR_INVALID_ARG;
    const size_t need = ws_bytes(N, P, E);
    if (ws_size < need || (need > 0 && (!ws || !aligned(ws, 16)))) return EP_ERR_INVALID_ARG;
    return hip_rc(launch_dispatch(topk_ids, N, P, *layout, sub_geom(N, P, E), static_cast<const int32_t *>(ws), phy_quota, log2phy, logcnt,
                                  slot_offsets, dispatch_pos, dispatch_src, as_stream(stream)));
}

int ep_replica_grad_reduce(float *native_grads, int64_t elems_per_expert, const float *slot_grads,
                           const int32_t *log2phy, const int32_t *logcnt, const ep_layout_t *layout,
                           ep_stream_t stream) {
    if (!layout_ok(layout) || !log2phy || !logcnt || elems_per_expert <= 0 || elems_per_expert % 4 != 0)
        return EP_ERR_INVALID_ARG;
    if (!native_grads || !aligned(native_grads, 16)) return EP_ERR_INVALID_ARG;
    if (layout->num_spare > 0 && (!slot_grads || !aligned(slot_grads, 16))) return EP_ERR_INVALID_ARG;
    if (layout->num_experts > kMaxPlans || layout->max_replicas > 64) return EP_ERR_INVALID_ARG;
    return hip_rc(launch_grad_reduce(native_grads, elems_per_expert, slot_grads, log2phy, logcnt, *layout,
                                     as_stream(stream)));
}

size_t ep_slot_fill_workspace_bytes(const ep_layout_t *layout) {
    if (!layout_ok(layout)) return 0;
    return fill_ws_bytes(layout->num_spare);
}

int ep_slot_fill(const void *expert_weights, int64_t bytes_per_expert, const int32_t *phy2log,
                 const ep_layout_t *layout, void *slot_buf, void *ws, size_t ws_size, ep_stream_t stream) {
    if (!layout_ok(layout) || !phy2log || bytes_per_expert <= 0 || bytes_per_expert % 16 != 0)
        return EP_ERR_INVALID_ARG;
    if (layout->num_spare == 0) return EP_OK;
    if (!expert_weights || !slot_buf || !aligned(expert_weights, 16) || !aligned(slot_buf, 16))
        return EP_ERR_INVALID_ARG;
    if (layout->num_spare > kMaxPlans) return EP_ERR_INVALID_ARG;
    // a workspace is optional; one too small, or misaligned, is an error
    const size_t need = fill_ws_bytes(layout->num_spare);
    if (ws && (ws_size < need || !aligned(ws, 16))) return EP_ERR_INVALID_ARG;
    int32_t *list = ws && need > 0 ? static_cast<int32_t *>(ws) : nullptr;
    return hip_rc(launch_slot_fill(expert_weights, bytes_per_expert, phy2log, *layout, slot_buf, list,
                                   as_stream(stream)));
}

int ep_balance_stats(const int32_t *load, const int32_t *phy_quota, int32_t P,
                     const ep_layout_t *layout, int64_t *stats, double *imbalance,
                     int32_t *rank_load, ep_stream_t stream) {
    if (!layout_ok(layout) || !load || !phy_quota || !stats || !imbalance) return EP_ERR_INVALID_ARG;
    if (P < 1 || P > kMaxPlans || !aligned(stats, 8) || !aligned(imbalance, 8)) return EP_ERR_INVALID_ARG;
    return hip_rc(launch_stats(load, phy_quota, P, *layout, stats, imbalance, rank_load,
                               as_stream(stream)));
}

const char *ep_status_string(int code) {
    switch (code) {
        case EP_OK: return "EP_OK";
        case EP_ERR_INVALID_ARG: return "EP_ERR_INVALID_ARG";
        case EP_ERR_HIP: return "EP_ERR_HIP";
        case EP_ERR_TOO_LARGE: return "EP_ERR_TOO_LARGE";
        default: return "EP_UNKNOWN";
    }
}

}  // extern "C"
