/*
 * ep_balance.h -- real-time MoE expert load balancing on one AMD MI355X (gfx950).
 *
 * The calls follow the problem as the UltraEP pages state it:
 *   - the gate emits top-k *logical* expert IDs per token; experts run as
 *     *physical* instances: each expert's native instance plus copies placed
 *     in a fixed number of reserved spare slots per EP rank, with no runtime
 *     allocation (UltraEP news article, m.youleyou.com, section on the key
 *     designs; UltraEP digest, agihunt.info, "What UltraEP does");
 *   - balancing reads the exact load after the gate, then solves how much load
 *     (a quota) every expert instance receives, jointly with where replicas go
 *     (UltraEP article, key designs, control-plane paragraph);
 *   - tokens of one logical expert are rerouted over its instances (same
 *     section, forward-pass paragraph); the three mapping tables are those of
 *     EPLB: physical slot -> logical expert, logical expert -> replica slots,
 *     replica count per expert (EPLB tutorial, t6page.pages.dev, section on the
 *     mapping tables);
 *   - replica weights are gathered into slot buffers that every layer reuses
 *     (UltraEP article, key designs, memory paragraph);
 *   - imbalance = load of the most loaded rank / mean rank load (UltraEP
 *     digest, "Reported results"); balancedness = its reciprocal (EPLB
 *     tutorial, measured-speedup section).
 *
 * All EP ranks of one layer are simulated on one GPU: the rank is an array
 * axis.  One "plan" is one (microbatch, layer); calls take P plans at once.
 *
 * Departures from the plain five-call sketch of this interface: the layout is
 * one packed device table built by ep_layout_init; ep_plan_quota also returns
 * each plan's move count; ep_balance_stats returns four int64 columns plus the
 * two imbalances as doubles (the move count and the step-cap flag come from
 * the planner); ep_route_noalloc serves callers that cannot allocate.
 *
 * Conventions shared by every call
 *   - Pointers named as device data are device pointers owned by the caller;
 *     the library allocates and frees nothing.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *     null stream) and returns; it never synchronises.  Calls on different
 *     streams are safe when their outputs do not alias.
 *   - The return value reports errors detectable on the host:
 *       EP_OK, EP_ERR_INVALID_ARG (null/misaligned pointer, bad size, workspace
 *       too small, unsupported shape), EP_ERR_HIP (a HIP runtime call failed).
 *     Data errors found on the device never force a sync: they are reported
 *     in the per-plan status words (EP_STATUS_*).
 *   - Integer work throughout; results do not depend on scheduling (no
 *     order-dependent atomics), so every output is bit-reproducible.
 */
#ifndef EP_BALANCE_H
#define EP_BALANCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *ep_stream_t; /* a hipStream_t */

enum {
    EP_OK = 0,
    EP_ERR_INVALID_ARG = -1,
    EP_ERR_HIP = -2,
    EP_ERR_TOO_LARGE = -3, /* ep_route_noalloc: the batch needs more than its scratch */
};

/* bits of the per-plan status word */
enum {
    EP_STATUS_BAD_ID = 1u,   /* an expert ID >= E was seen; such pairs count nowhere */
    EP_STATUS_STEP_CAP = 2u, /* the planner stopped at its step cap                  */
    EP_STATUS_BAD_LOAD = 4u, /* the planner got a load < 0 or a total above INT32_MAX */
};

/*
 * Physical layout of one EP group: native placement + spare slots per rank.
 *
 * Physical slots are numbered rank-major; inside rank r the native experts come
 * first in ascending logical ID, then the rank's spare slots.  The o-th spare
 * slot in that order owns row o of the slot buffer.
 *
 * `tables` points to device memory holding ep_layout_table_ints() int32 values
 * written by ep_layout_init(); the struct itself lives in host memory and is
 * read by every call at enqueue time.
 */
typedef struct ep_layout {
    int32_t num_experts;  /* E: logical experts                                   */
    int32_t num_ranks;    /* R: EP ranks                                          */
    int32_t num_phys;     /* Phi = E + S physical slots                           */
    int32_t num_spare;    /* S: spare slots over all ranks                        */
    int32_t max_replicas; /* rho = min(R, 1 + S): row width of log2phy            */
    int32_t max_rank_natives; /* most native experts on one rank                  */
    int32_t max_rank_spares;  /* most spare slots on one rank                     */
    int32_t ranks_per_domain; /* D > 0: replicas stay in the scale-up domain of     */
                              /* their expert's native rank (rank r is in domain    */
                              /* r / D; an 8-GPU xGMI node on MI355X); 0: anywhere. */
                              /* ep_layout_init sets 0; the caller may change it.   */
    const int32_t *tables;/* device, packed tables (see ep_layout_init)           */
} ep_layout_t;

/* Number of int32 values ep_layout_init writes for (E, R, S). */
size_t ep_layout_table_ints(int32_t num_experts, int32_t num_ranks, int32_t num_spare);

/*
 * Validate a placement, pack its tables on the host and copy them with a
 * blocking hipMemcpy into `device_tables` (caller-owned, at least
 * ep_layout_table_ints(E, R, sum(spare_count)) int32 values).  Fills *out.
 *   native_count  host [R]: native experts of each rank (>= 0, sum = E)
 *   native_experts host [E]: rank-major lists, rank r's block of native_count[r]
 *                  IDs in any order (each logical ID exactly once)
 *   spare_count   host [R]: spare slots of each rank (>= 0)
 * Setup only (once per EP group), not part of the per-plan path.
 * Returns EP_ERR_INVALID_ARG for an invalid placement or a rank count above
 * EP_MAX_RANKS, EP_ERR_HIP if the copy fails.
 */
#define EP_MAX_RANKS 4096
#define EP_MAX_EXPERTS 16384
int ep_layout_init(int32_t num_experts, int32_t num_ranks, const int32_t *native_count,
                   const int32_t *native_experts, const int32_t *spare_count,
                   int32_t *device_tables, size_t device_table_ints, ep_layout_t *out);

/*
 * Workspace for one (ep_load_histogram, ep_reroute) pair, in bytes.  It carries
 * per-expert pair counts from the histogram to the reroute (and the dispatch
 * layout): for every sub-block of consecutive pairs, how many pairs of each
 * expert come before it in the plan, stored as a count within a segment of
 * sub-blocks plus a per-segment base.  With E <= 256 it also holds a one-byte
 * copy of every ID and a flag per sub-block (padding or IDs >= E present),
 * which the reroute reads in place of the int32 IDs of unflagged sub-blocks.
 * Pass the same buffer, untouched in between, with the same N and P.  Grows
 * as P * (sub-blocks + segments + 1) * (E + 1) * 4, about 1/8 to 1/4 byte per
 * pair, plus about 1 byte per pair with E <= 256.
 */
size_t ep_workspace_bytes(int64_t pairs_per_plan, int32_t num_plans, int32_t num_experts);

/*
 * Pairs per sub-block for a launch of P plans of N pairs with E experts: the
 * unit of work of one wave in the histogram, the reroute and the dispatch
 * layout, and the unit of the workspace's count rows (one row of E + 1 int32
 * per sub-block).  A power of two from 1024 up; 0 for invalid sizes.  For
 * callers that account for the workspace's traffic; no call needs it.
 */
int64_t ep_sub_block_pairs(int64_t pairs_per_plan, int32_t num_plans, int32_t num_experts);

/*
 * A1 -- exact per-expert load of every plan (UltraEP article, key designs:
 * the global load is read after the gate and before dispatch).
 *   topk_ids  device int32 [P][N]: N = R*T*k pairs per plan in (source rank,
 *             token, k) order.  ID < 0 is padding (ignored); ID >= E is an
 *             error: status bit EP_STATUS_BAD_ID, the pair is ignored.
 *   load      device int32 [P][E] (written)
 *   ws        device, >= ep_workspace_bytes(N, P, E) bytes, 16-byte aligned
 *   status    device uint32 [P] (written: EP_STATUS_BAD_ID or 0)
 * N may be 0 (loads become 0).  Requires N < 2^31, 1 <= P <= 65535 and
 * E <= 5119 (eight LDS histograms of E + 1 counters in a workgroup's 160 KiB).
 */
int ep_load_histogram(const int32_t *topk_ids, int64_t pairs_per_plan, int32_t num_plans,
                      const ep_layout_t *layout, int32_t *load, void *ws, size_t ws_bytes,
                      uint32_t *status, ep_stream_t stream);

/*
 * A2 -- joint replica placement and per-instance quotas, one independent plan
 * per (microbatch, layer) starting from the native placement (UltraEP article,
 * key designs: each exploration step may create a replica and move load; the
 * pages do not print the solver, so the rule below is this library's reading).
 *
 * Greedy, capped at 2*S + R committed moves (status EP_STATUS_STEP_CAP):
 *   h = most loaded rank (lowest index on ties); candidates = loaded instances
 *   on h by (quota desc, expert asc).  First try to re-level a candidate that
 *   already has replicas, else replicate one onto the least loaded rank (lowest
 *   index on ties) that has a free spare slot and no instance of it, into that
 *   rank's lowest free spare slot.  Every move water-fills the expert's load
 *   over its instances: with other-expert loads b_i sorted by (b, rank), the m*
 *   largest-prefix instances with m*b_(m) < load + sum_{j<=m} b_(j) end at
 *   floor(S/m*) or one more (the extra units to the first S mod m* of them).
 *   With layout->ranks_per_domain = D > 0 the replica rank must also share the
 *   expert's native domain (UltraEP article, section on why it reaches the
 *   optimum: replication stays inside the high-bandwidth scale-up domain).
 *   A move is kept only if it lowers h's load; the loop stops when no move
 *   does.  Replicas left with quota 0 are freed.
 *   load      device int32 [P][E]
 *   phy2log   device int32 [P][Phi]: logical expert of each slot, -1 = empty
 *   phy_quota device int32 [P][Phi]: pairs each instance receives (0 if empty)
 *   logcnt    device int32 [P][E]: instances per expert (>= 1)
 *   log2phy   device int32 [P][E][rho]: instance slots in ascending order, -1 padded
 *   steps     device int32 [P] or NULL: committed moves
 *   status    device uint32 [P] or NULL: EP_STATUS_STEP_CAP and
 *             EP_STATUS_BAD_LOAD are OR-ed in
 * Every load must be >= 0 and a plan's total at most INT32_MAX (true of any
 * histogram of fewer than 2^31 pairs).  A plan that breaks this makes no move:
 * it keeps the native placement (quota = load) and gets EP_STATUS_BAD_LOAD.
 * Requires rho <= 64 (at most 64 instances of one expert), 1 <= P <= 65535,
 * and either R <= 64 with at most 8 natives and 16 spare slots per rank, or
 * tables that fit the generic kernel's 160 KiB of LDS (about 60 bytes per rank
 * and per expert: R = E up to about 2700); other layouts return
 * EP_ERR_INVALID_ARG.
 */
int ep_plan_quota(const int32_t *load, int32_t num_plans, const ep_layout_t *layout,
                  int32_t *phy2log, int32_t *phy_quota, int32_t *logcnt, int32_t *log2phy,
                  int32_t *steps, uint32_t *status, ep_stream_t stream);

/*
 * A3 -- order-preserving reroute of every (token,k) pair to a physical instance
 * of its own logical expert (UltraEP article, key designs: reroute splits one
 * native expert's tokens over its replicas; EPLB tutorial: the physical ID is
 * looked up from the top-k logical ID).  The j-th pair (0-based, flat order)
 * of expert e goes to the instance i (ascending slot order) with
 * Q_i <= j < Q_i + quota_i, Q_i the sum of the quotas of the instances before i.
 *   topk_ids  device int32 [P][N], the same IDs the histogram saw (with
 *             E <= 256 most pairs are read from the workspace's byte copy;
 *             pairs are read here only in sub-blocks that hold padding or bad
 *             IDs, where phys_ids is not 16-byte aligned, and after a
 *             sub-block's last whole 256-pair tile)
 *   phy_quota, log2phy, logcnt: a plan as ep_plan_quota writes it (each
 *             instance a distinct slot in [0, Phi), logcnt in [0, rho])
 *   ws        the workspace filled by ep_load_histogram for these IDs
 *   phys_ids  device int32 [P][N] (written): physical slot, -1 for padding,
 *             invalid IDs and pairs beyond the expert's total quota
 * phys_ids 4-byte aligned.  LDS bounds the shape: 16 E + 8 Phi + 256 bytes
 * must fit 160 KiB (E up to about 6800 at Phi = E); otherwise, and for a ws
 * smaller than ep_workspace_bytes(N, P, E), EP_ERR_INVALID_ARG.
 */
int ep_reroute(const int32_t *topk_ids, int64_t pairs_per_plan, int32_t num_plans,
               const ep_layout_t *layout, const int32_t *phy_quota, const int32_t *log2phy,
               const int32_t *logcnt, const void *ws, size_t ws_bytes, int32_t *phys_ids,
               ep_stream_t stream);

/*
 * A1 -> A2 -> A3 over a batch of plans (e.g. every MoE layer of a microbatch)
 * cut into chunks that overlap across three streams: one planner launch lasts
 * about as long as its slowest plan, so the planner of chunk c runs while the
 * histogram of chunk c + 1 streams, and the reroute of chunk c while the
 * planner of chunk c + 1 runs.  The outputs are exactly those of
 * ep_load_histogram, ep_plan_quota and ep_reroute made in order on one stream
 * (arguments and layouts as there, P plans).  Kernels of two streams run side
 * by side only when the streams sit on different hardware queues; the HIP
 * runtime spreads streams over its queues (GPU_MAX_HW_QUEUES of them, 4 by
 * default) in creation order, so three streams created one after another get
 * three queues, whereas a side stream that shares the queue of the caller's
 * busy stream loses the overlap.
 *   chunk_plans  host int32 [num_chunks]: plans per chunk, each >= 1, summing
 *                to P; 1 <= num_chunks <= EP_MAX_CHUNKS
 *   ws           device, >= ep_pipeline_workspace_bytes(N, chunk_plans,
 *                num_chunks, E) bytes, 16-byte aligned: one histogram
 *                workspace per chunk
 *   stream       the caller's stream: the chain starts after the work already
 *                enqueued there and later work there waits for all of it
 *   side_streams host array of three distinct streams of the caller, none of
 *                them `stream`, default priority: histograms run on [0],
 *                planners on [1], reroutes on [2]
 *   events       2 + 2 * num_chunks events of the caller (hipEvent_t, e.g.
 *                created with hipEventDisableTiming), recorded and waited on
 *                here; no other work may use them until the chain completes
 * Returns EP_ERR_INVALID_ARG (nothing enqueued) for bad arguments, including
 * any that one of the three calls would reject for a chunk.
 */
#define EP_MAX_CHUNKS 16
size_t ep_pipeline_workspace_bytes(int64_t pairs_per_plan, const int32_t *chunk_plans, int32_t num_chunks,
                                   int32_t num_experts);
int ep_route_pipelined(const int32_t *topk_ids, int64_t pairs_per_plan, int32_t num_plans,
                       const ep_layout_t *layout, const int32_t *chunk_plans, int32_t num_chunks,
                       int32_t *load, uint32_t *status, int32_t *phy2log, int32_t *phy_quota,
                       int32_t *logcnt, int32_t *log2phy, int32_t *steps, int32_t *phys_ids, void *ws,
                       size_t ws_bytes, ep_stream_t stream, const ep_stream_t *side_streams,
                       void *const *events);

/*
 * Next row after A3 -- dispatch layout for the token all-to-all (EPLB
 * tutorial, EPLB / DeepEP section: dispatch sends each pair to its physical
 * replica; combine gathers results back to the logical expert).  Pairs are
 * laid out physical-slot-major: slot s owns positions [off_s, off_s + quota_s)
 * with off the exclusive prefix of the quotas in slot order, and the j-th pair
 * of expert e, served by the instance whose quota range starts at Q, sits at
 * off_s + (j - Q): for plans whose quotas cover the loads, the stable counting
 * sort of the pairs by physical slot.
 *   topk_ids, plan tables, ws  as for ep_reroute (the same histogram workspace)
 *   slot_offsets  device int32 [P][Phi+1] (written): off_s, last entry = total
 *   dispatch_pos  device int32 [P][N] (written): position of each pair, -1 for
 *                 padding, invalid IDs and pairs past the expert's quotas
 *   dispatch_src  device int32 [P][N] (written): pair index (within the plan)
 *                 at each position, -1 for positions no pair takes
 * All output arrays 4-byte aligned.  LDS bounds the shape: 24 E + 12 Phi + 20
 * bytes must fit 160 KiB (about E <= 4500 at Phi = E).
 */
int ep_dispatch_layout(const int32_t *topk_ids, int64_t pairs_per_plan, int32_t num_plans,
                       const ep_layout_t *layout, const int32_t *phy_quota, const int32_t *log2phy,
                       const int32_t *logcnt, const void *ws, size_t ws_bytes,
                       int32_t *slot_offsets, int32_t *dispatch_pos, int32_t *dispatch_src,
                       ep_stream_t stream);

/*
 * A4 -- weight distribution on one GPU: gather the weights of every expert that
 * occupies a spare slot into that slot's row of the cross-layer slot buffer
 * (UltraEP article, key designs: reserved slots, weight buffers reused across
 * layers).  One plan (one layer) per call; empty spare slots are not written.
 * Each distinct expert is read once (with a workspace: once per group of up to
 * 4 of its slots) and stored into every slot that holds it.
 *   expert_weights device [E][bytes_per_expert], one layer (16-byte aligned)
 *   phy2log        device int32 [Phi], that layer's plan
 *   slot_buf       device [S][bytes_per_expert] (16-byte aligned)
 *   ws             device, ep_slot_fill_workspace_bytes(layout) bytes (16-byte
 *                  aligned), or NULL: with it the call first lists the plan's
 *                  distinct experts and their slots there (a one-workgroup
 *                  kernel) and then streams each expert's weights in address
 *                  order, the faster form; without it every workgroup finds
 *                  its slot's expert itself.  The workspace holds no state
 *                  between calls; calls in flight at once need their own.
 * bytes_per_expert must be a positive multiple of 16.  A spare slot whose
 * phy2log entry lies outside [0, E) is empty: its row is not written.
 */
size_t ep_slot_fill_workspace_bytes(const ep_layout_t *layout);
int ep_slot_fill(const void *expert_weights, int64_t bytes_per_expert, const int32_t *phy2log,
                 const ep_layout_t *layout, void *slot_buf, void *ws, size_t ws_bytes,
                 ep_stream_t stream);

/*
 * Next row -- replica gradient reduction in backward (UltraEP article, key
 * designs: replicas keep no optimizer state and their gradients are reduced
 * back to the native expert; backward paragraph: accumulation keeps a fixed
 * order so the reduction is deterministic).  One plan (one layer) per call:
 * for every expert with logcnt >= 2, its native row becomes the fp32 fold of
 * its instances' gradient rows in ascending physical-slot order
 *     acc = g(inst 0); acc = acc + g(inst 1); ...
 * reading native_grads[e] for the native instance and slot_grads[o] for the
 * replica in the o-th spare slot.  Other rows and slot_grads are not written.
 *   native_grads device float [E][n] (in/out), 16-byte aligned
 *   slot_grads   device float [S][n], the gradient half of the slot buffer
 *   log2phy, logcnt  that layer's plan (ep_plan_quota)
 * n = elems_per_expert must be a positive multiple of 4; requires rho <= 64 and
 * E <= 65535.  Rows of experts whose instance list names a slot outside
 * [0, Phi) are left unchanged.
 */
int ep_replica_grad_reduce(float *native_grads, int64_t elems_per_expert, const float *slot_grads,
                           const int32_t *log2phy, const int32_t *logcnt, const ep_layout_t *layout,
                           ep_stream_t stream);

/*
 * A5 -- balance statistics per plan (UltraEP digest, "Reported results":
 * most loaded rank over the mean).
 *   stats      device int64 [P][4]: max rank load before (native placement),
 *              max rank load after (sum of quotas per rank), total load,
 *              replicas in use (spare slots with a positive quota)
 *   imbalance  device double [P][2]: before, after = max * R / total (exactly
 *              rounded; 1.0 when total == 0)
 *   rank_load  device int32 [P][2][R] or NULL: per-rank loads before / after
 */
int ep_balance_stats(const int32_t *load, const int32_t *phy_quota, int32_t num_plans,
                     const ep_layout_t *layout, int64_t *stats, double *imbalance,
                     int32_t *rank_load, ep_stream_t stream);

/*
 * For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): ep_load_histogram,
 * ep_plan_quota and ep_reroute in one call, with the workspace that carries
 * the histogram's per-sub-block counts (and byte copy) to the reroute held in
 * a device array of the library instead of a caller buffer.  The outputs are
 * exactly those of the three calls (same arguments, same meaning, same
 * layouts; status is written as the histogram writes it, then the planner's
 * flag is OR-ed in).  The call allocates nothing and never synchronises.
 *
 * The array is EP_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held by every GPU
 * the library runs this call on until the process ends.  A batch whose
 * workspace, ep_workspace_bytes(N, P, E), is larger returns EP_ERR_TOO_LARGE
 * and enqueues nothing; 64 MiB holds, for example, 14 plans of 4.2M pairs at
 * E = 128 (a plan = one layer of an EP64 group with 8192 tokens per rank,
 * top-8) or 75 such plans at E = 384.  All argument checks of the three calls run before
 * anything is enqueued.  Every call on one GPU shares that GPU's array, so
 * calls whose work overlaps on one GPU (other streams, other host threads)
 * race and corrupt each other's results: serialise them (one stream, or
 * events) on each GPU.
 */
#define EP_NOALLOC_SCRATCH_BYTES (64u << 20)
int ep_route_noalloc(const int32_t *topk_ids, int64_t pairs_per_plan, int32_t num_plans,
                     const ep_layout_t *layout, int32_t *load, uint32_t *status, int32_t *phy2log,
                     int32_t *phy_quota, int32_t *logcnt, int32_t *log2phy, int32_t *steps,
                     int32_t *phys_ids, ep_stream_t stream);

/* Human-readable name of a return code. */
const char *ep_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* EP_BALANCE_H */
