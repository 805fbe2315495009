// ep_route_noalloc: the histogram -> plan -> reroute chain for callers that
// cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  It runs the same kernels as
// ep_load_histogram, ep_plan_quota and ep_reroute, but the workspace that
// carries the per-sub-block counts (and, with E <= 256, the one-byte ID copy)
// from the histogram to the reroute is a file-scope device array of fixed
// size instead of a caller buffer.
//
// In host code the array's name is only a host-side stand-in for the symbol;
// its device address is looked up once per device with hipGetSymbolAddress
// (each GPU holds its own copy at its own address) and only that address is
// passed to the kernels.
#include <mutex>

#include "ep_internal.h"

using namespace ep;

namespace {

constexpr size_t kScratchBytes = (size_t)EP_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_ptr[kMaxDevices];  // device address of `scratch` per device, set once

// Device address of this device's scratch array, or null on failure.
void *scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" int ep_route_noalloc(const int32_t *topk_ids, int64_t N, int32_t P, const ep_layout_t *layout,
                                int32_t *load, uint32_t *status, int32_t *phy2log, int32_t *phy_quota,
                                int32_t *logcnt, int32_t *log2phy, int32_t *steps, int32_t *phys_ids,
                                ep_stream_t stream) {
    if (!layout || layout->num_experts < 1 || N < 0 || P < 1 || P > 65535) return EP_ERR_INVALID_ARG;
    const int E = layout->num_experts;
    if (ws_bytes(N, P, E) > kScratchBytes) return EP_ERR_TOO_LARGE;
    void *ws = scratch_ptr();
    if (!ws) return EP_ERR_HIP;
    // every check of the three calls before anything is enqueued
    int rc = check_histogram(topk_ids, N, P, layout, load, ws, kScratchBytes, status);
    if (rc == EP_OK) rc = check_plan(load, P, layout, phy2log, phy_quota, logcnt, log2phy);
    if (rc == EP_OK) rc = check_reroute(topk_ids, N, P, layout, phy_quota, log2phy, logcnt, ws, kScratchBytes,
                                        phys_ids);
    if (rc != EP_OK) return rc;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const SubGeom g = sub_geom(N, P, E);
    const Compact cp = compact_of(ws, N, P, E);
    hipError_t err = launch_histogram(topk_ids, N, P, E, g, static_cast<int32_t *>(ws), cp, load, status, s);
    if (err == hipSuccess)
        err = launch_plan(load, P, *layout, phy2log, phy_quota, logcnt, log2phy, steps, status, s,
                          plan_lanes_cfg(*layout));
    if (err == hipSuccess)
        err = launch_reroute(topk_ids, N, P, *layout, g, static_cast<const int32_t *>(ws), cp, phy_quota,
                             log2phy, logcnt, phys_ids, s);
    return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}
