// A2: joint replica placement + per-instance quotas (UltraEP news article,
// section on the key designs: the solver works out how much load each expert
// instance receives, and each exploration step may both instantiate a replica
// and update the load distribution; the load lives in fixed spare slots).
//
// One wave (one workgroup of 64 lanes) per plan; plans of many layers and
// microbatches run side by side in one launch.  Two kernels: the generic one
// below keeps all state in LDS (rank loads, free spare counts, slot owners and
// quotas, per-expert instance counts) and takes any R; the rank-per-lane one
// further down keeps each rank's state in its lane's registers (R <= 64) and
// is the one the workloads here use.  Both make the same moves.
// Each step:
//   1. hottest rank h   = wave max of the packed key (load << 32 | ~rank);
//   2. candidates       = loaded instances on h, visited in descending
//                         (quota << 32 | ~expert) order by repeated wave max;
//   3. re-level pass    (experts that already have a replica), then a
//      replicate pass   (destination = wave max of (~load << 32 | ~rank) over
//                         ranks with a free spare and no instance of the expert);
//   4. water-fill       of the expert's load over its instances: instances sit
//                         one per lane, are ranked by (background, rank) with a
//                         64-way count, the sorted backgrounds go through a wave
//                         prefix sum, and a ballot finds the filled prefix m*.
// A move is committed only when it lowers h's load.  Integer arithmetic only.
#include "ep_internal.h"

// Phase marks of the rank-per-lane planner for a profiling build only
// (-DEP_PLAN_PHASES, see plan_phases.py beside the package): lane 0 accumulates
// s_memtime stamps per phase of a move and, at the end, writes them per plan
// to a device array that ep_plan_phases_read copies out.  In the normal build
// the marks compile to nothing.
#ifdef EP_PLAN_PHASES
#define EP_PHASE_COUNT 8
#define EP_PHASE_PLANS 256
static __device__ unsigned long long ep_phase_buf[EP_PHASE_PLANS][16];
#define EP_PHASE_DECL unsigned long long ph_acc_[EP_PHASE_COUNT] = {0, 0, 0, 0, 0, 0, 0, 0}, ph_t_ = 0, ph_t0_ = __builtin_amdgcn_s_memtime(), ph_tries_ = 0, ph_rank_ = 0;
#define EP_PHASE_START() ph_t_ = __builtin_amdgcn_s_memtime();
#define EP_PHASE(k)                                                        \
    {                                                                      \
        const unsigned long long t_ = __builtin_amdgcn_s_memtime();        \
        ph_acc_[k] += t_ - ph_t_;                                          \
        ph_t_ = t_;                                                        \
    }
#define EP_PHASE_COUNT_TRY() ph_tries_++;
#define EP_PHASE_COUNT_RANK() ph_rank_++;
#define EP_PHASE_LOOP_END() const unsigned long long ph_tl_ = __builtin_amdgcn_s_memtime();
#define EP_PHASE_WRITE(p, lane, moves)                                                          \
    if ((lane) == 0 && (p) < EP_PHASE_PLANS) {                                                  \
        for (int k_ = 0; k_ < EP_PHASE_COUNT; k_++) ep_phase_buf[p][k_] = ph_acc_[k_];          \
        ep_phase_buf[p][8] = ph_tries_;                                                         \
        ep_phase_buf[p][9] = ph_rank_;                                                          \
        ep_phase_buf[p][10] = (unsigned long long)(moves);                                      \
        ep_phase_buf[p][11] = ph_tl_ - ph_t0_;                                                  \
        ep_phase_buf[p][12] = __builtin_amdgcn_s_memtime() - ph_tl_;                            \
    }
#else
#define EP_PHASE_DECL
#define EP_PHASE_START()
#define EP_PHASE(k)
#define EP_PHASE_COUNT_TRY()
#define EP_PHASE_COUNT_RANK()
#define EP_PHASE_LOOP_END()
#define EP_PHASE_WRITE(p, lane, moves)
#endif

namespace ep {
namespace {

struct PlanArgs {
    int32_t E, R, Phi, S, rho;
    int32_t D;  // ranks per scale-up domain (0: no constraint)
    Tables T;
};

__device__ __forceinline__ uint32_t inv(uint32_t x) { return 0xffffffffu - x; }

__global__ __launch_bounds__(kWave) void plan_kernel_generic(const int32_t *__restrict__ load, PlanArgs a,
                                                     int32_t *__restrict__ phy2log,
                                                     int32_t *__restrict__ phy_quota,
                                                     int32_t *__restrict__ logcnt,
                                                     int32_t *__restrict__ log2phy,
                                                     int32_t *__restrict__ steps_out,
                                                     uint32_t *__restrict__ status) {
    const int E = a.E, R = a.R, Phi = a.Phi, S = a.S, rho = a.rho;
    extern __shared__ __align__(16) unsigned char sh_raw[];
    uint64_t *emask = reinterpret_cast<uint64_t *>(sh_raw);  // [E]
    int64_t *sbuf = reinterpret_cast<int64_t *>(emask + E);  // [64]
    int32_t *rl = reinterpret_cast<int32_t *>(sbuf + kWave);  // [R]  rank load
    int32_t *freec = rl + R;                                   // [R]  free spare slots
    int32_t *rfirst = freec + R;                               // [R+1]
    int32_t *rnat = rfirst + R + 1;                            // [R]
    int32_t *stamp = rnat + R;                                 // [R]
    int32_t *owner = stamp + R;                                // [Phi]
    int32_t *quota = owner + Phi;                              // [Phi]
    int32_t *srank = quota + Phi;                              // [Phi]
    int32_t *hslot = srank + Phi;                              // [E]
    int32_t *ld = hslot + E;                                   // [E]
    int32_t *icnt = ld + E;                                    // [E]
    int32_t *erun = icnt + E;                                  // [E]
    int32_t *nshift = erun + E;                                // [E]
    int32_t *sslot = nshift + E;                               // [S]
    int32_t *islot = sslot + S;                                // [64]

    const int p = blockIdx.x;
    const int lane = threadIdx.x;
    const int32_t *lp = load + (int64_t)p * E;

    for (int r = lane; r <= R; r += kWave) rfirst[r] = a.T.rank_first[r];
    for (int r = lane; r < R; r += kWave) { rnat[r] = a.T.rank_nat[r]; stamp[r] = -1; }
    for (int s = lane; s < Phi; s += kWave) { owner[s] = a.T.slot_home[s]; srank[s] = a.T.slot_rank[s]; }
    // loads must be >= 0 with a total that fits int32 (every quota and rank
    // load is then a partial sum of them); a plan that breaks this is flagged
    // and keeps its native placement
    int64_t lsum = 0;
    bool lneg = false;
    for (int e = lane; e < E; e += kWave) {
        hslot[e] = a.T.home_slot[e];
        const int32_t v = lp[e];
        ld[e] = v;
        icnt[e] = 1;
        lsum += v;
        lneg |= v < 0;
    }
    const bool bad_load = __ballot(lneg) != 0 || readlane_i64(wave_incl_scan_i64(lsum), kWave - 1) > 0x7fffffffLL;
    for (int o = lane; o < S; o += kWave) sslot[o] = a.T.spare_slot[o];
    __syncthreads();
    for (int s = lane; s < Phi; s += kWave) {
        const int e = owner[s];
        quota[s] = e >= 0 ? ld[e] : 0;
    }
    __syncthreads();
    for (int r = lane; r < R; r += kWave) {
        int sum = 0;
        for (int s = rfirst[r]; s < rfirst[r + 1]; s++) sum += quota[s];
        rl[r] = sum;
        freec[r] = rfirst[r + 1] - rfirst[r] - rnat[r];
    }
    __syncthreads();

    int tries = 0;
    const uint64_t lt = lanemask_lt();

    // Water-fill expert e over its instances (plus a new one on the least loaded
    // eligible rank when `replicate`); commit if h's load drops below Lh.
    auto try_move = [&](int e, bool replicate, int h, int64_t Lh) -> bool {
        // instances: native in lane 0, replicas compacted after it
        if (lane == 0) islot[0] = hslot[e];
        int n = 1;
        for (int base = 0; base < S; base += kWave) {
            const int o = base + lane;
            int s = -1;
            bool own = false;
            if (o < S) { s = sslot[o]; own = owner[s] == e; }
            const uint64_t m = __ballot(own);
            if (own) islot[n + __popcll(m & lt)] = s;
            n += __popcll(m);
        }
        __syncthreads();
        int d = -1;
        if (replicate) {
            tries++;
            if (lane < n) stamp[srank[islot[lane]]] = tries;
            __syncthreads();
            uint64_t best = 0;
            const int hr = srank[hslot[e]];
            for (int r = lane; r < R; r += kWave) {
                if (freec[r] > 0 && stamp[r] != tries && (a.D == 0 || r / a.D == hr / a.D)) {
                    const uint64_t k = ((uint64_t)inv((uint32_t)rl[r]) << 32) | inv((uint32_t)r);
                    best = k > best ? k : best;
                }
            }
            best = wave_max_u64(best);
            if (best == 0) return false;
            d = (int)inv((uint32_t)best);
            n += 1;
        }
        int my_r = 0, my_q = 0, my_s = -1;
        if (lane < n) {
            if (replicate && lane == n - 1) {
                my_r = d;
                my_s = rfirst[d] + rnat[d] + (rfirst[d + 1] - rfirst[d] - rnat[d] - freec[d]);
            } else {
                my_s = islot[lane];
                my_r = srank[my_s];
                my_q = quota[my_s];
            }
        }
        const int64_t my_b = (lane < n) ? (int64_t)rl[my_r] - my_q : 0;
        const uint64_t my_key = ((uint64_t)my_b << 32) | (uint32_t)my_r;
        int pos = 0;
        for (int j = 0; j < n; j++) {
            const uint64_t kj = (uint64_t)readlane_i64((int64_t)my_key, j);
            pos += kj < my_key ? 1 : 0;
        }
        if (lane < n) sbuf[pos] = my_b;
        __syncthreads();
        const int64_t bs = (lane < n) ? sbuf[lane] : 0;
        const int64_t Sm = (int64_t)ld[e] + wave_incl_scan_i64(bs);
        const uint64_t cm = __ballot(lane < n && (int64_t)(lane + 1) * bs < Sm);
        const int mstar = cm ? 64 - __clzll((long long)cm) : 0;
        int64_t base = 0, rem = 0;
        if (mstar > 0) {
            const int64_t Ss = readlane_i64(Sm, mstar - 1);
            base = Ss / mstar;
            rem = Ss - (int64_t)mstar * base;
        }
        int64_t my_nq = 0;
        if (lane < n && pos < mstar) my_nq = base - my_b + (pos < rem ? 1 : 0);
        const uint64_t hm = __ballot(lane < n && my_r == h);
        const int hl = __ffsll((long long)hm) - 1;
        const int64_t newLh = readlane_i64(my_b + my_nq, hl);
        __syncthreads();
        if (newLh >= Lh) return false;
        if (lane < n) {
            quota[my_s] = (int32_t)my_nq;
            rl[my_r] = (int32_t)(my_b + my_nq);
        }
        if (replicate && lane == n - 1) {
            owner[my_s] = e;
            freec[d] -= 1;
            icnt[e] += 1;
        }
        __syncthreads();
        return true;
    };

    const int cap = 2 * S + R;
    int steps = 0, cap_hit = 0;
    for (; !bad_load;) {
        if (steps == cap) { cap_hit = 1; break; }
        uint64_t key = 0;
        for (int r = lane; r < R; r += kWave) {
            const uint64_t k = ((uint64_t)(uint32_t)rl[r] << 32) | inv((uint32_t)r);
            key = k > key ? k : key;
        }
        key = wave_max_u64(key);
        const int h = (int)inv((uint32_t)key);
        const int64_t Lh = (int64_t)(key >> 32);
        const int f0 = rfirst[h], nh = rfirst[h + 1] - f0;

        bool committed = false;
        for (int pass = 0; pass < 2 && !committed; pass++) {
            uint64_t prev = ~0ull;
            for (;;) {
                uint64_t best = 0;
                for (int i = lane; i < nh; i += kWave) {
                    const int s = f0 + i;
                    const int e = owner[s];
                    const int q = quota[s];
                    if (e >= 0 && q > 0 && (pass == 1 || icnt[e] >= 2)) {
                        const uint64_t k = ((uint64_t)(uint32_t)q << 32) | inv((uint32_t)e);
                        if (k < prev && k > best) best = k;
                    }
                }
                best = wave_max_u64(best);
                if (best == 0) break;
                prev = best;
                const int e = (int)inv((uint32_t)best);
                if (try_move(e, pass == 1, h, Lh)) { committed = true; break; }
            }
        }
        if (!committed) break;
        steps++;
    }

    // replicas left without load are freed; natives always stay
    for (int o = lane; o < S; o += kWave) {
        const int s = sslot[o];
        if (owner[s] >= 0 && quota[s] == 0) owner[s] = -1;
    }
    for (int e = lane; e < E; e += kWave) { emask[e] = 0; erun[e] = 0; nshift[e] = 0; }
    __syncthreads();

    int32_t *o_p2l = phy2log + (int64_t)p * Phi;
    int32_t *o_q = phy_quota + (int64_t)p * Phi;
    for (int s = lane; s < Phi; s += kWave) { o_p2l[s] = owner[s]; o_q[s] = quota[s]; }
    int32_t *o_l2p = log2phy + (int64_t)p * E * rho;
    for (int64_t i = lane; i < (int64_t)E * rho; i += kWave) o_l2p[i] = -1;
    __syncthreads();

    // position of each replica among its expert's instances (ascending slots):
    // spare slots are visited in ascending order 64 at a time; an LDS bit mask
    // per expert gives the rank inside the group, a per-expert counter the
    // count of earlier groups
    for (int base = 0; base < S; base += kWave) {
        const int o = base + lane;
        int s = -1, e = -1;
        if (o < S) { s = sslot[o]; e = owner[s]; }
        if (e >= 0) atomicOr(reinterpret_cast<unsigned long long *>(&emask[e]), 1ull << lane);
        __syncthreads();
        uint64_t m = 0;
        int run = 0;
        if (e >= 0) { m = emask[e]; run = erun[e]; }
        __syncthreads();
        if (e >= 0) {
            const uint64_t below = m & lt;
            if (below == 0) { erun[e] = run + __popcll(m); emask[e] = 0; }
            const int hs = hslot[e];
            const int pos = run + __popcll(below) + (hs < s ? 1 : 0);
            if (pos < rho) o_l2p[(int64_t)e * rho + pos] = s;
            if (hs > s) atomicAdd(&nshift[e], 1);
        }
        __syncthreads();
    }
    for (int e = lane; e < E; e += kWave) {
        const int ns = nshift[e];
        if (ns < rho) o_l2p[(int64_t)e * rho + ns] = hslot[e];
        logcnt[(int64_t)p * E + e] = 1 + erun[e];
    }
    if (lane == 0) {
        if (steps_out) steps_out[p] = steps;
        const uint32_t flags = (cap_hit ? (uint32_t)EP_STATUS_STEP_CAP : 0u) | (bad_load ? (uint32_t)EP_STATUS_BAD_LOAD : 0u);
        if (status && flags) status[p] |= flags;
    }
}


// ---------------------------------------------------------------------------
// Rank-per-lane planner (R <= 64, at most NPR native experts and SPR spare
// slots per rank).
//
// Lane r owns rank r.  In registers: its load, free spare count, its native
// experts (ID, load, quota, instance count) and its spare slots (owner,
// quota, and the owner's native rank, index and load).  Candidates on the
// hottest rank come from that lane's registers by readlane; the instances of an expert are found lane-locally (its native
// lane, or a lane holding it in a spare slot); the water-fill runs over the
// lanes that host the expert and a commit only touches their registers.  LDS
// holds the static (native rank, native index) of every expert, a per-expert
// flag that says whether a re-level could change the expert's quotas (set
// when a commit moves the load of a rank that hosts it, cleared when the
// expert itself is levelled; candidates whose flag is clear are not tried in
// the re-level pass), and, at the end, the per-expert masks of replica ranks
// used to order log2phy.
// ---------------------------------------------------------------------------
// v[i] (v[0] for i outside [0, N)) from registers.  Built from masks rather
// than selects: the compiler turns a chain of selects between elements into
// one indexed load, which keeps the whole array in scratch memory.
template <int N>
__device__ __forceinline__ int32_t pick(const int32_t (&v)[N], int i) {
    int32_t r = v[0] & -(int32_t)(i < 1 || i >= N);
#pragma unroll
    for (int k = 1; k < N; k++) r |= v[k] & -(int32_t)(i == k);
    return r;
}

template <int NPR, int SPR>
__global__ __launch_bounds__(kWave) void plan_kernel_lanes(const int32_t *__restrict__ load, PlanArgs a,
                                                           int32_t *__restrict__ phy2log,
                                                           int32_t *__restrict__ phy_quota,
                                                           int32_t *__restrict__ logcnt,
                                                           int32_t *__restrict__ log2phy,
                                                           int32_t *__restrict__ steps_out,
                                                           uint32_t *__restrict__ status) {
    const int E = a.E, R = a.R, Phi = a.Phi, S = a.S, rho = a.rho;
    extern __shared__ __align__(16) unsigned char sh_raw[];
    uint64_t *emask = reinterpret_cast<uint64_t *>(sh_raw);      // [E] ranks of live replicas
    int32_t *nri = reinterpret_cast<int32_t *>(emask + E);       // [E] native rank << 8 | index
    // [E + 1] set when a move of another expert changed the load of a rank that
    // hosts this expert after the expert was last water-filled; re-levelling
    // an expert that is not set would reproduce its current quotas, so such
    // candidates are skipped
    int32_t *edirty = nri + E;

    const int p = blockIdx.x;
    const int lane = threadIdx.x;
    const int32_t *lp = load + (int64_t)p * E;
    EP_PHASE_DECL

    const bool is_rank = lane < R;
    const uint64_t rank_mask = R >= kWave ? ~0ull : ((1ull << R) - 1);
    const int f0 = is_rank ? a.T.rank_first[lane] : 0;
    const int nat = is_rank ? a.T.rank_nat[lane] : 0;
    const int spc = is_rank ? a.T.rank_first[lane + 1] - f0 - nat : 0;
    int freec = spc;
    int32_t nat_e[NPR], nat_ld[NPR], nat_q[NPR], nat_ic[NPR];
    // a spare slot's owner and quota, and the owner's native rank << 8 | index
    // and load (copied when the replica is made)
    int32_t sp_owner[SPR], sp_q[SPR], sp_nri[SPR], sp_ld[SPR];
#pragma unroll
    for (int i = 0; i < NPR; i++) nat_e[i] = i < nat ? a.T.slot_home[f0 + i] : -1;
#pragma unroll
    for (int i = 0; i < NPR; i++) {
        nat_ld[i] = nat_e[i] >= 0 ? lp[nat_e[i]] : 0;
        nat_q[i] = nat_ld[i];
        nat_ic[i] = 1;
        if (nat_e[i] >= 0) nri[nat_e[i]] = (lane << 8) | i;
    }
#pragma unroll
    for (int j = 0; j < SPR; j++) { sp_owner[j] = -1; sp_q[j] = 0; sp_nri[j] = 0; sp_ld[j] = 0; }
    for (int e = lane; e <= E; e += kWave) edirty[e] = 0;  // entry E stays clear: empty slots read it
    for (int e = lane; e < E; e += kWave) emask[e] = 0;
    int rl = 0;
    int64_t lsum = 0;
    bool lneg = false;
#pragma unroll
    for (int i = 0; i < NPR; i++) {
        rl += nat_ld[i];
        lsum += nat_ld[i];
        lneg |= nat_ld[i] < 0;
    }
    // loads must be >= 0 with a total that fits int32 (every quota and rank
    // load is then a partial sum of them); a plan that breaks this is flagged
    // and keeps its native placement
    const bool bad_load = __ballot(lneg) != 0 || readlane_i64(wave_incl_scan_i64(lsum), kWave - 1) > 0x7fffffffLL;
    __syncthreads();

    // lane i: floor((2^32 - 1) / (i + 1)), for the water-fill's division by m*
    const uint32_t rcp_m = 0xffffffffu / (uint32_t)(lane + 1);
    const int cap = 2 * S + R;
    int steps = 0, cap_hit = 0;
    for (; !bad_load;) {
        if (steps == cap) { cap_hit = 1; break; }
        EP_PHASE_START()
        // The hottest rank's loaded instance slots are the candidates (slot
        // k < NPR its k-th native, NPR + j its j-th spare).  A pass tries them
        // in descending (quota, -expert) order, each found when needed (most
        // steps commit on the first one): the largest quota left, the lowest
        // expert among equal quotas (the experts of one rank are distinct).
        // With few slots per rank the slots are read into scalar registers and
        // compared there (no wave reduction: Qwen3-like plans 3.5 % faster);
        // with more, one slot per lane and a wave reduction per pick (a
        // scalar pick over 8 slots was 2 % slower).
        constexpr int K = NPR + SPR;
        constexpr bool kScalarPick = K <= 5;
        uint32_t db = 0;
        if constexpr (kScalarPick) {
            // re-level flags of this lane's slots (LDS reads issued ahead of
            // the reduction, which hides their latency)
#pragma unroll
            for (int i = 0; i < NPR; i++) db |= (edirty[nat_e[i] >= 0 ? nat_e[i] : E] != 0 ? 1u : 0u) << i;
#pragma unroll
            for (int j = 0; j < SPR; j++)
                db |= (edirty[sp_owner[j] >= 0 ? sp_owner[j] : E] != 0 ? 1u : 0u) << (NPR + j);
        }
        // hottest rank (lowest index on ties)
        const int vmax = wave_max_i32(is_rank ? rl : -1);
        // (a ballot of one compare, masked in scalar registers, saves turning
        // a combined condition into a vector value and back)
        const int h = __ffsll((long long)(__ballot(rl == vmax) & rank_mask)) - 1;
        const int Lh = vmax;
        EP_PHASE(0)

        uint64_t vm, relevel;        // loaded slots; those worth a re-level (replicated, flag set)
        uint32_t sq[kScalarPick ? K : 1];
        int32_t se[kScalarPick ? K : 1];
        int ce = -1, cq = 0, cld = 0, cpk = 0;  // lane k: slot k's expert, quota, load, native
        if constexpr (kScalarPick) {
            uint32_t vb = 0, rb = 0;
#pragma unroll
            for (int i = 0; i < NPR; i++) {
                vb |= (nat_q[i] > 0 ? 1u : 0u) << i;
                rb |= (nat_ic[i] >= 2 ? 1u : 0u) << i;
            }
#pragma unroll
            for (int j = 0; j < SPR; j++) {
                vb |= (sp_q[j] > 0 ? 1u : 0u) << (NPR + j);
                rb |= 1u << (NPR + j);
            }
            rb &= vb & db;
            vm = (uint32_t)__builtin_amdgcn_readlane((int)vb, h);
            relevel = (uint32_t)__builtin_amdgcn_readlane((int)rb, h);
#pragma unroll
            for (int i = 0; i < NPR; i++) {
                sq[i] = (uint32_t)__builtin_amdgcn_readlane(nat_q[i], h);
                se[i] = __builtin_amdgcn_readlane(nat_e[i], h);
            }
#pragma unroll
            for (int j = 0; j < SPR; j++) {
                sq[NPR + j] = (uint32_t)__builtin_amdgcn_readlane(sp_q[j], h);
                se[NPR + j] = __builtin_amdgcn_readlane(sp_owner[j], h);
            }
        } else {
            int cic = 2;
#pragma unroll
            for (int i = 0; i < NPR; i++) {
                const int e = __builtin_amdgcn_readlane(nat_e[i], h);
                const int q = __builtin_amdgcn_readlane(nat_q[i], h);
                const int l = __builtin_amdgcn_readlane(nat_ld[i], h);
                const int ic = __builtin_amdgcn_readlane(nat_ic[i], h);
                if (lane == i) { ce = e; cq = q; cld = l; cic = ic; cpk = (h << 8) | i; }
            }
#pragma unroll
            for (int j = 0; j < SPR; j++) {
                const int e = __builtin_amdgcn_readlane(sp_owner[j], h);
                const int q = __builtin_amdgcn_readlane(sp_q[j], h);
                const int pk = __builtin_amdgcn_readlane(sp_nri[j], h);
                const int l = __builtin_amdgcn_readlane(sp_ld[j], h);
                if (lane == NPR + j) { ce = e; cq = q; cpk = pk; cld = l; }
            }
            const bool valid = ce >= 0 && cq > 0;
            const int cdirty = valid ? edirty[ce] : 0;
            vm = __ballot(valid);
            relevel = __ballot(valid && cic >= 2 && cdirty != 0);
        }
        EP_PHASE(1)

        bool committed = false;
        for (int pass = relevel ? 0 : 1; pass < 2 && !committed; pass++) {
            uint64_t left = pass == 0 ? relevel : vm;
            while (left && !committed) {
                int e, nr, idx, T;
                if constexpr (kScalarPick) {
                    int bk = 0;
                    uint32_t bq = 0;
                    e = 0x7fffffff;
#pragma unroll
                    for (int k = 0; k < K; k++) {
                        const bool better = ((left >> k) & 1u) && (sq[k] > bq || (sq[k] == bq && se[k] < e));
                        bk = better ? k : bk;
                        bq = better ? sq[k] : bq;
                        e = better ? se[k] : e;
                    }
                    left &= ~(1ull << bk);
                    if (bk < NPR) {
                        nr = h;
                        idx = bk;
                        T = __builtin_amdgcn_readlane(pick(nat_ld, bk), h);
                    } else {
                        const int pk = __builtin_amdgcn_readlane(pick(sp_nri, bk - NPR), h);
                        nr = pk >> 8;
                        idx = pk & 0xff;
                        T = __builtin_amdgcn_readlane(pick(sp_ld, bk - NPR), h);
                    }
                } else {
                    const bool in = (left >> lane) & 1;
                    const int qmax = wave_max_i32(in ? cq : -1);
                    uint64_t tm = __ballot(cq == qmax) & left;
                    if (tm & (tm - 1)) {
                        const bool tie = (tm >> lane) & 1;
                        const int emin = wave_min_i32(tie ? ce : 0x7fffffff);
                        tm &= __ballot(ce == emin);
                    }
                    const int cl = __ffsll((long long)tm) - 1;
                    left &= ~(1ull << cl);
                    e = __builtin_amdgcn_readlane(ce, cl);
                    const int pk = __builtin_amdgcn_readlane(cpk, cl);
                    nr = pk >> 8;
                    idx = pk & 0xff;
                    T = __builtin_amdgcn_readlane(cld, cl);
                }
                const bool replicate = pass == 1;
                EP_PHASE_COUNT_TRY()
                EP_PHASE(2)

                // instances of e on this lane's rank
                const bool nat_here = lane == nr;
                int jr = -1;
#pragma unroll
                for (int j = 0; j < SPR; j++)
                    if (j < spc && sp_owner[j] == e) jr = j;
                int q = 0;
#pragma unroll
                for (int j = 0; j < SPR; j++)
                    if (j == jr) q = sp_q[j];
                if (nat_here) q = pick(nat_q, idx);
                const bool inst = nat_here || jr >= 0;
                const int b = rl - q;
                bool isnew = false;
                if (replicate) {
                    const bool elig = is_rank && freec > 0 && !inst && (a.D == 0 || lane / a.D == nr / a.D);
                    const int vmin = wave_min_i32(elig ? rl : 0x7fffffff);
                    const uint64_t em = __ballot(elig && rl == vmin);
                    if (em == 0) continue;
                    isnew = lane == __ffsll((long long)em) - 1;
                }
                const bool act = inst || isnew;
                EP_PHASE(3)
                // sorted position by (background, rank) and inclusive prefix sum
                int pos = 0;
                uint32_t Sinc = (uint32_t)T;
                for (uint64_t mm = __ballot(act); mm; mm &= mm - 1) {
                    const int j = __ffsll((long long)mm) - 1;
                    const int bj = __builtin_amdgcn_readlane(b, j);
                    const bool less = bj < b || (bj == b && j < lane);
                    pos += less ? 1 : 0;
                    if (less || j == lane) Sinc += (uint32_t)bj;
                    EP_PHASE_COUNT_RANK()
                }
                EP_PHASE(4)
                // the filled instances form a prefix of the sorted order, so
                // m* = number of instances with m*b_(m) < S_m
                const int mstar = __popcll(__ballot(act && (uint64_t)(pos + 1) * (uint32_t)b < Sinc));
                int qn = 0;
                if (mstar > 0) {
                    const int ls = __ffsll((long long)__ballot(act && pos == mstar - 1)) - 1;
                    const uint32_t Ss = (uint32_t)__builtin_amdgcn_readlane((int)Sinc, ls);
                    // Ss / m* from the reciprocal held by lane m* - 1: the
                    // high word of Ss * floor((2^32 - 1) / m*) is the
                    // quotient or one less (Ss < 2^32), one step corrects it
                    const uint32_t um = (uint32_t)mstar;
                    uint32_t base = __umulhi(Ss, (uint32_t)__builtin_amdgcn_readlane((int)rcp_m, mstar - 1));
                    uint32_t rem = Ss - um * base;
                    if (rem >= um) {
                        base += 1;
                        rem -= um;
                    }
                    if (act && pos < mstar) qn = (int)base - b + ((uint32_t)pos < rem ? 1 : 0);
                }
                const int newLh = __builtin_amdgcn_readlane(act ? b + qn : rl, h);
                EP_PHASE(5)
                if (newLh >= Lh) continue;
                // commit (lane-local)
                if (act) rl = b + qn;
                if (nat_here) {
                    // (value selects, not stores under a condition, for the
                    // same reason as in pick)
#pragma unroll
                    for (int i = 0; i < NPR; i++) {
                        nat_q[i] = i == idx ? qn : nat_q[i];
                        nat_ic[i] += (i == idx && replicate) ? 1 : 0;
                    }
                }
#pragma unroll
                for (int j = 0; j < SPR; j++)
                    if (j == jr) sp_q[j] = qn;
                if (isnew) {
                    const int jn = spc - freec;
#pragma unroll
                    for (int j = 0; j < SPR; j++)
                        if (j == jn) { sp_owner[j] = e; sp_q[j] = qn; sp_nri[j] = (nr << 8) | idx; sp_ld[j] = T; }
                    freec -= 1;
                }
                // every expert on a rank whose load moved needs a new level,
                // except the one just levelled
                if (act) {
#pragma unroll
                    for (int i = 0; i < NPR; i++)
                        if (i < nat) edirty[nat_e[i]] = 1;
#pragma unroll
                    for (int j = 0; j < SPR; j++)
                        if (j < spc && sp_owner[j] >= 0) edirty[sp_owner[j]] = 1;
                }
                wave_lds_fence();
                if (lane == 0) edirty[e] = 0;
                committed = true;
                EP_PHASE(6)
            }
        }
        EP_PHASE(7)
        if (!committed) break;
        steps++;
    }
    EP_PHASE_LOOP_END()

    // replicas left without load are freed; record each live replica's rank
#pragma unroll
    for (int j = 0; j < SPR; j++) {
        if (j < spc && sp_owner[j] >= 0 && sp_q[j] == 0) sp_owner[j] = -1;
        if (j < spc && sp_owner[j] >= 0)
            atomicOr(reinterpret_cast<unsigned long long *>(&emask[sp_owner[j]]), 1ull << lane);
    }
    int32_t *o_p2l = phy2log + (int64_t)p * Phi;
    int32_t *o_q = phy_quota + (int64_t)p * Phi;
    int32_t *o_l2p = log2phy + (int64_t)p * E * rho;
    for (int64_t i = lane; i < (int64_t)E * rho; i += kWave) o_l2p[i] = -1;   // coalesced padding
    __syncthreads();

    const uint64_t below_me = (1ull << lane) - 1;
#pragma unroll
    for (int i = 0; i < NPR; i++) {
        if (i < nat) {
            const int e = nat_e[i];
            const int s = f0 + i;
            const uint64_t m = emask[e];
            o_p2l[s] = e;
            o_q[s] = nat_q[i];
            logcnt[(int64_t)p * E + e] = 1 + __popcll(m);
            o_l2p[(int64_t)e * rho + __popcll(m & below_me)] = s;
        }
    }
#pragma unroll
    for (int j = 0; j < SPR; j++) {
        if (j < spc) {
            const int s = f0 + nat + j;
            const int e = sp_owner[j];
            o_p2l[s] = e;
            o_q[s] = e >= 0 ? sp_q[j] : 0;
            if (e >= 0) {
                const int nr = nri[e] >> 8;
                const int pos = __popcll(emask[e] & below_me) + (nr < lane ? 1 : 0);
                o_l2p[(int64_t)e * rho + pos] = s;
            }
        }
    }
    if (lane == 0) {
        if (steps_out) steps_out[p] = steps;
        const uint32_t flags = (cap_hit ? (uint32_t)EP_STATUS_STEP_CAP : 0u) | (bad_load ? (uint32_t)EP_STATUS_BAD_LOAD : 0u);
        if (status && flags) status[p] |= flags;
    }
    EP_PHASE_WRITE(p, lane, steps)
}

}  // namespace

size_t plan_lds_bytes(const ep_layout_t &L) {
    const size_t E = L.num_experts, R = L.num_ranks, Phi = L.num_phys, S = L.num_spare;
    return 8 * E + 8 * kWave + 4 * (5 * R + 1 + 3 * Phi + 5 * E + S + kWave);
}

static size_t lanes_lds_bytes(const ep_layout_t &L) { return (size_t)L.num_experts * 16 + 16; }

static int pow2_at_least(int x) {
    int v = 1;
    while (v < x) v <<= 1;
    return v;
}

int plan_lanes_cfg(const ep_layout_t &L) {
    if (L.num_ranks > kWave) return 0;
    // natives per rank in registers: 1, 2, 4, 6 or 8 (6 saves a quarter of the
    // work for layouts with 5 or 6 natives per rank)
    const int mn = L.max_rank_natives > 0 ? L.max_rank_natives : 1;
    const int npr = (mn > 4 && mn <= 6) ? 6 : pow2_at_least(mn);
    const int spr = pow2_at_least(L.max_rank_spares > 0 ? L.max_rank_spares : 1);
    if (npr > 8 || spr > 16 || lanes_lds_bytes(L) > kLdsMax) return 0;
    return npr * 32 + spr;
}

#define EP_LANES_CASE(NP, SP)                                                                   \
    case NP * 32 + SP:                                                                          \
        hipLaunchKernelGGL((plan_kernel_lanes<NP, SP>), g, b, lds, s, load, a, phy2log, phy_quota, \
                           logcnt, log2phy, steps, status);                                     \
        break;
#define EP_LANES_ROW(NP) EP_LANES_CASE(NP, 1) EP_LANES_CASE(NP, 2) EP_LANES_CASE(NP, 4) \
    EP_LANES_CASE(NP, 8) EP_LANES_CASE(NP, 16)

hipError_t launch_plan(const int32_t *load, int32_t P, const ep_layout_t &L, int32_t *phy2log,
                       int32_t *phy_quota, int32_t *logcnt, int32_t *log2phy, int32_t *steps,
                       uint32_t *status, hipStream_t s, int cfg) {
    PlanArgs a{L.num_experts, L.num_ranks, L.num_phys, L.num_spare, L.max_replicas, L.ranks_per_domain,
               tables_of(L)};
    const dim3 g((unsigned)P), b(kWave);
    const size_t lds = lanes_lds_bytes(L);
    switch (cfg) {
        EP_LANES_ROW(1)
        EP_LANES_ROW(2)
        EP_LANES_ROW(4)
        EP_LANES_ROW(6)
        EP_LANES_ROW(8)
        default:
            hipLaunchKernelGGL(plan_kernel_generic, g, b, plan_lds_bytes(L), s, load, a, phy2log,
                               phy_quota, logcnt, log2phy, steps, status);
            break;
    }
    return hipGetLastError();
}

}  // namespace ep

#ifdef EP_PLAN_PHASES
// Profiling build only: copies the per-plan phase cycles of the last planner
// launch (plans [0, P), P <= 256, 16 values each: 8 phases, tries, ranking
// iterations, moves, loop cycles, epilogue cycles) to host memory.
extern "C" int ep_plan_phases_read(unsigned long long *host, int P) {
    if (!host || P < 1 || P > EP_PHASE_PLANS) return EP_ERR_INVALID_ARG;
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(ep_phase_buf), (size_t)P * 16 * sizeof(unsigned long long), 0,
                               hipMemcpyDeviceToHost) == hipSuccess
               ? EP_OK
               : EP_ERR_HIP;
}
#endif
