// ep_route_pipelined: the histogram -> plan -> reroute chain over a batch of
// plans cut into chunks that overlap across three streams.  A planner launch
// lasts about as long as its slowest plan (one wave per plan), so a batch of
// layers planned in one launch leaves the streaming kernels idle meanwhile;
// cut into chunks, the planner of chunk c runs while the histogram of chunk
// c + 1 streams, and the reroute of chunk c while the planner of chunk c + 1
// runs.  Histograms, planners and reroutes each go on a side stream of their
// own, and the caller's stream only orders the chain against its other work:
// kernels overlap only across hardware queues, and three streams created one
// after another sit on three different queues, while a side stream could share
// the caller's (busy) one.  Each chunk has its own histogram workspace (a
// slice of the caller's buffer).  The outputs are those of the three calls
// made in order on one stream.  Host-side argument checks of every launch run
// before anything is enqueued.
#include "ep_internal.h"

using namespace ep;

namespace {

inline size_t chunk_ws_bytes(int64_t N, int32_t plans, int32_t E) { return align256(ws_bytes(N, plans, E)); }

}  // namespace

extern "C" size_t ep_pipeline_workspace_bytes(int64_t N, const int32_t *chunk_plans, int32_t num_chunks,
                                              int32_t E) {
    if (N < 0 || E < 1 || !chunk_plans || num_chunks < 1 || num_chunks > EP_MAX_CHUNKS) return 0;
    size_t total = 0;
    for (int c = 0; c < num_chunks; c++) {
        if (chunk_plans[c] < 1) return 0;
        total += chunk_ws_bytes(N, chunk_plans[c], E);
    }
    return total;
}

extern "C" int ep_route_pipelined(const int32_t *topk_ids, int64_t N, int32_t P, const ep_layout_t *layout,
                                  const int32_t *chunk_plans, int32_t num_chunks, int32_t *load,
                                  uint32_t *status, int32_t *phy2log, int32_t *phy_quota, int32_t *logcnt,
                                  int32_t *log2phy, int32_t *steps, int32_t *phys_ids, void *ws,
                                  size_t ws_size, ep_stream_t stream, const ep_stream_t *side_streams,
                                  void *const *events) {
    if (!layout || !chunk_plans || num_chunks < 1 || num_chunks > EP_MAX_CHUNKS || !events || N < 0 || P < 1)
        return EP_ERR_INVALID_ARG;
    if (!load || !status || !phy2log || !phy_quota || !logcnt || !log2phy) return EP_ERR_INVALID_ARG;
    if (N > 0 && (!topk_ids || !phys_ids)) return EP_ERR_INVALID_ARG;
    if (!side_streams) return EP_ERR_INVALID_ARG;
    for (int i = 0; i < 3; i++) {
        if (!side_streams[i] || side_streams[i] == stream) return EP_ERR_INVALID_ARG;
        for (int j = 0; j < i; j++)
            if (side_streams[j] == side_streams[i]) return EP_ERR_INVALID_ARG;
    }
    for (int i = 0; i < 2 + 2 * num_chunks; i++)
        if (!events[i]) return EP_ERR_INVALID_ARG;
    const int E = layout->num_experts, Phi = layout->num_phys, rho = layout->max_replicas;
    if (E < 1) return EP_ERR_INVALID_ARG;
    int64_t sum = 0;
    for (int c = 0; c < num_chunks; c++) {
        if (chunk_plans[c] < 1) return EP_ERR_INVALID_ARG;
        sum += chunk_plans[c];
    }
    if (sum != P) return EP_ERR_INVALID_ARG;
    const size_t need = ep_pipeline_workspace_bytes(N, chunk_plans, num_chunks, E);
    if (ws_size < need || !ws || ((uintptr_t)ws % 16) != 0) return EP_ERR_INVALID_ARG;

    // every launch's checks first, on the chunk's slices of the arrays
    {
        int64_t a = 0;
        size_t off = 0;
        for (int c = 0; c < num_chunks; c++) {
            const int32_t n = chunk_plans[c];
            void *w = static_cast<unsigned char *>(ws) + off;
            const size_t wb = chunk_ws_bytes(N, n, E);
            const int32_t *ids = N > 0 ? topk_ids + a * N : nullptr;
            int rc = check_histogram(ids, N, n, layout, load + a * E, w, wb, status + a);
            if (rc == EP_OK)
                rc = check_plan(load + a * E, n, layout, phy2log + a * Phi, phy_quota + a * Phi, logcnt + a * E,
                                log2phy + a * E * rho);
            if (rc == EP_OK)
                rc = check_reroute(ids, N, n, layout, phy_quota + a * Phi, log2phy + a * E * rho, logcnt + a * E,
                                   w, wb, N > 0 ? phys_ids + a * N : nullptr);
            if (rc != EP_OK) return rc;
            a += n;
            off += wb;
        }
    }

    const hipStream_t s0 = reinterpret_cast<hipStream_t>(stream);
    const hipStream_t sh = reinterpret_cast<hipStream_t>(side_streams[0]);
    const hipStream_t sp = reinterpret_cast<hipStream_t>(side_streams[1]);
    const hipStream_t sr = reinterpret_cast<hipStream_t>(side_streams[2]);
    hipEvent_t e_start = static_cast<hipEvent_t>(events[0]);
    hipEvent_t e_done = static_cast<hipEvent_t>(events[1]);
    auto e_hist = [&](int c) { return static_cast<hipEvent_t>(events[2 + c]); };
    auto e_plan = [&](int c) { return static_cast<hipEvent_t>(events[2 + num_chunks + c]); };
    const int cfg = plan_lanes_cfg(*layout);

#define EP_TRY(x)                                     \
    do {                                              \
        if ((x) != hipSuccess) return EP_ERR_HIP;     \
    } while (0)
    // the side streams start after the work already on the caller's stream
    EP_TRY(hipEventRecord(e_start, s0));
    EP_TRY(hipStreamWaitEvent(sh, e_start, 0));
    EP_TRY(hipStreamWaitEvent(sp, e_start, 0));
    EP_TRY(hipStreamWaitEvent(sr, e_start, 0));
    int64_t a = 0;
    size_t off = 0;
    for (int c = 0; c < num_chunks; c++) {
        const int32_t n = chunk_plans[c];
        int32_t *w = reinterpret_cast<int32_t *>(static_cast<unsigned char *>(ws) + off);
        EP_TRY(launch_histogram(N > 0 ? topk_ids + a * N : nullptr, N, n, E, sub_geom(N, n, E), w, compact_of(w, N, n, E),
                                load + a * E, status + a, sh));
        EP_TRY(hipEventRecord(e_hist(c), sh));
        a += n;
        off += chunk_ws_bytes(N, n, E);
    }
    a = 0;
    for (int c = 0; c < num_chunks; c++) {
        const int32_t n = chunk_plans[c];
        EP_TRY(hipStreamWaitEvent(sp, e_hist(c), 0));
        EP_TRY(launch_plan(load + a * E, n, *layout, phy2log + a * Phi, phy_quota + a * Phi, logcnt + a * E,
                           log2phy + a * E * rho, steps ? steps + a : nullptr, status + a, sp, cfg));
        EP_TRY(hipEventRecord(e_plan(c), sp));
        a += n;
    }
    a = 0;
    off = 0;
    for (int c = 0; c < num_chunks; c++) {
        const int32_t n = chunk_plans[c];
        int32_t *w = reinterpret_cast<int32_t *>(static_cast<unsigned char *>(ws) + off);
        EP_TRY(hipStreamWaitEvent(sr, e_plan(c), 0));
        EP_TRY(launch_reroute(N > 0 ? topk_ids + a * N : nullptr, N, n, *layout, sub_geom(N, n, E), w,
                              compact_of(w, N, n, E), phy_quota + a * Phi, log2phy + a * E * rho, logcnt + a * E,
                              N > 0 ? phys_ids + a * N : nullptr, sr));
        a += n;
        off += chunk_ws_bytes(N, n, E);
    }
    // later work on the caller's stream waits for the last reroute
    EP_TRY(hipEventRecord(e_done, sr));
    EP_TRY(hipStreamWaitEvent(s0, e_done, 0));
#undef EP_TRY
    return EP_OK;
}
