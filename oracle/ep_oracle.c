/*
 * CPU oracle for real-time MoE expert load balancing -- TEST INFRASTRUCTURE.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The product path (the HIP library) never calls it and
 * shares no code, header or table with it.
 *
 * Plain, slow, single-threaded C.  Every routine follows a passage of the
 * source pages:
 *   [UltraEP-1] UltraEP news article (m.youleyou.com), section on the key
 *               designs ("关键设计"): reserved spare slots per rank, global
 *               load read after the gate, per-instance quota solving where each
 *               exploration step may both create a replica and move load,
 *               reroute splitting one expert's tokens over its replicas.
 *   [UltraEP-4] UltraEP digest (agihunt.info), "What UltraEP does" and
 *               "Reported results": imbalance = most loaded rank / mean load.
 *   [EPLB-5]    EPLB tutorial (t6page.pages.dev), redundant-expert section and
 *               the three mapping tables (physical expert per GPU slot, replica
 *               indices per logical expert, replica count per logical expert).
 *
 * Where the pages leave a step open the plainest reading is taken:
 *   - one (token,k) pair is one unit of load; a rank's load is the sum of the
 *     quotas of the instances it hosts;
 *   - physical slots are numbered rank-major; inside a rank the native experts
 *     come first in ascending logical ID, then the rank's spare slots;
 *   - a replica goes into the lowest free spare slot of its rank, and a rank
 *     never hosts two instances of one expert;
 *   - the instances of an expert are ordered by ascending physical slot;
 *   - the planner is the greedy "re-level, else replicate" loop below, with
 *     water-filled integer quotas, highest load first and lowest index on ties,
 *     capped at 2*S + R committed moves; replicas left with quota 0 are freed;
 *   - the j-th pair (0-based, flat (rank, token, k) order) of an expert goes to
 *     the instance whose quota range [Q_i, Q_i + q_i) holds j;
 *   - IDs < 0 are padding; IDs >= E are errors, treated like padding.
 *
 * Parity pins for every routine live in tests/test_oracle_*.py.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_BAD_LAYOUT -1
#define OR_NO_MEMORY -2

/* ------------------------------------------------------------------------- */
/* Layout: native placement plus spare slots per rank.                       */
/* ------------------------------------------------------------------------- */
typedef struct {
    int E, R, Phi, S;
    int *first_slot;   /* [R+1] first physical slot of each rank            */
    int *nat_cnt;      /* [R]                                               */
    int *spare_cnt;    /* [R]                                               */
    int *slot_home;    /* [Phi] native expert of a slot, -1 for spare slots */
    int *slot_rank;    /* [Phi]                                             */
    int *home_slot;    /* [E]   the native slot of each expert              */
    int *spare_slot;   /* [S]   physical slot of the o-th spare slot        */
} layout_t;

static void layout_free(layout_t *L) {
    free(L->first_slot); free(L->nat_cnt); free(L->spare_cnt); free(L->slot_home);
    free(L->slot_rank); free(L->home_slot); free(L->spare_slot);
    memset(L, 0, sizeof(*L));
}

/* Build the slot numbering from the per-rank native lists (rank-major, E
 * entries in total) and the per-rank spare counts. */
static int layout_build(layout_t *L, int E, int R, const int32_t *native_count,
                        const int32_t *native_experts, const int32_t *spare_count) {
    memset(L, 0, sizeof(*L));
    if (E <= 0 || R <= 0) return OR_BAD_LAYOUT;
    int total_nat = 0, total_spare = 0;
    for (int r = 0; r < R; r++) {
        if (native_count[r] < 0 || spare_count[r] < 0) return OR_BAD_LAYOUT;
        total_nat += native_count[r];
        total_spare += spare_count[r];
    }
    if (total_nat != E) return OR_BAD_LAYOUT;
    L->E = E; L->R = R; L->S = total_spare; L->Phi = E + total_spare;
    L->first_slot = calloc((size_t)R + 1, sizeof(int));
    L->nat_cnt = calloc((size_t)R, sizeof(int));
    L->spare_cnt = calloc((size_t)R, sizeof(int));
    L->slot_home = calloc((size_t)L->Phi, sizeof(int));
    L->slot_rank = calloc((size_t)L->Phi, sizeof(int));
    L->home_slot = calloc((size_t)E, sizeof(int));
    L->spare_slot = calloc((size_t)(total_spare > 0 ? total_spare : 1), sizeof(int));
    if (!L->first_slot || !L->nat_cnt || !L->spare_cnt || !L->slot_home || !L->slot_rank ||
        !L->home_slot || !L->spare_slot) { layout_free(L); return OR_NO_MEMORY; }
    for (int e = 0; e < E; e++) L->home_slot[e] = -1;

    int slot = 0, in = 0, o = 0;
    for (int r = 0; r < R; r++) {
        L->first_slot[r] = slot;
        L->nat_cnt[r] = native_count[r];
        L->spare_cnt[r] = spare_count[r];
        /* natives of this rank in ascending logical ID (insertion sort) */
        int n = native_count[r];
        int *tmp = malloc((size_t)(n > 0 ? n : 1) * sizeof(int));
        if (!tmp) { layout_free(L); return OR_NO_MEMORY; }
        for (int i = 0; i < n; i++) {
            int v = native_experts[in + i], j = i;
            while (j > 0 && tmp[j - 1] > v) { tmp[j] = tmp[j - 1]; j--; }
            tmp[j] = v;
        }
        for (int i = 0; i < n; i++) {
            int e = tmp[i];
            if (e < 0 || e >= E || L->home_slot[e] != -1) { free(tmp); layout_free(L); return OR_BAD_LAYOUT; }
            L->home_slot[e] = slot;
            L->slot_home[slot] = e;
            L->slot_rank[slot] = r;
            slot++;
        }
        free(tmp);
        in += n;
        for (int i = 0; i < spare_count[r]; i++) {
            L->slot_home[slot] = -1;
            L->slot_rank[slot] = r;
            L->spare_slot[o++] = slot;
            slot++;
        }
    }
    L->first_slot[R] = slot;
    return OR_OK;
}

/* ------------------------------------------------------------------------- */
/* A1: exact per-expert load of one plan [UltraEP-1: the global load is read */
/* after the gate; UltraEP-4: the actual token load after the gate].         */
/* ------------------------------------------------------------------------- */
int or_histogram(const int32_t *ids, int64_t n, int32_t E, int32_t *load, int64_t *num_bad) {
    int64_t bad = 0;
    for (int32_t e = 0; e < E; e++) load[e] = 0;
    for (int64_t i = 0; i < n; i++) {
        int32_t v = ids[i];
        if (v < 0) continue;              /* padding */
        if (v >= E) { bad++; continue; }  /* invalid ID: flagged, not counted */
        load[v] += 1;
    }
    if (num_bad) *num_bad = bad;
    return OR_OK;
}

/* ------------------------------------------------------------------------- */
/* Water-filling of one expert's load over its instances.                    */
/*                                                                           */
/* Instance i sits on a rank whose load without this expert is b_i (the      */
/* "background").  The expert's T units are poured onto the lowest          */
/* backgrounds first until they meet one level: with backgrounds sorted by   */
/* (b asc, rank asc), the m* filled instances are the largest prefix with    */
/* m*b_(m) < T + b_(1) + ... + b_(m); they end at floor(S/m*) or one more,   */
/* the extra unit going to the first (S mod m*) of them in sorted order.     */
/* ------------------------------------------------------------------------- */
static void waterfill(int64_t T, int n, const int64_t *b, const int *rank, int64_t *q) {
    int *ord = malloc((size_t)n * sizeof(int));
    for (int i = 0; i < n; i++) {               /* insertion sort by (b, rank) */
        int j = i;
        while (j > 0 && (b[ord[j - 1]] > b[i] || (b[ord[j - 1]] == b[i] && rank[ord[j - 1]] > rank[i]))) {
            ord[j] = ord[j - 1];
            j--;
        }
        ord[j] = i;
    }
    int mstar = 0;
    int64_t S = T, Sstar = 0;
    for (int m = 1; m <= n; m++) {
        S += b[ord[m - 1]];
        if ((int64_t)m * b[ord[m - 1]] < S) { mstar = m; Sstar = S; }
    }
    for (int i = 0; i < n; i++) q[i] = 0;
    if (mstar > 0) {
        int64_t base = Sstar / mstar, rem = Sstar - (int64_t)mstar * base;
        for (int j = 0; j < mstar; j++) {
            int i = ord[j];
            q[i] = base - b[i] + (j < rem ? 1 : 0);
        }
    }
    free(ord);
}

/* ------------------------------------------------------------------------- */
/* A2: joint replica placement + per-instance quota [UltraEP-1: quota per    */
/* expert instance; each exploration step can create a replica and update    */
/* the load distribution; fixed spare slots per rank; EPLB-5: three tables]. */
/* ------------------------------------------------------------------------- */
typedef struct { int slot; int expert; int64_t quota; } cand_t;

/* ranks_per_domain D > 0 confines replicas to the scale-up domain of the
 * expert's native rank (rank r lies in domain r / D) [UltraEP article, section
 * on why it reaches the optimum: hot-expert replication stays inside the
 * high-bandwidth scale-up domain]; D = 0 places replicas anywhere. */
/* Loads must be >= 0 with a total that fits int32 (the widths of the tables);
 * a plan that breaks this makes no move and keeps the native placement, and
 * *bad_load_out is set. */
int or_plan_domain(int32_t E, int32_t R, const int32_t *native_count, const int32_t *native_experts,
                   const int32_t *spare_count, const int32_t *load,
                   int32_t *phy2log, int32_t *phy_quota, int32_t *logcnt, int32_t *log2phy,
                   int32_t rho, int32_t ranks_per_domain, int32_t *steps_out, int32_t *cap_hit_out,
                   int32_t *bad_load_out) {
    layout_t L;
    int rc = layout_build(&L, E, R, native_count, native_experts, spare_count);
    if (rc != OR_OK) return rc;
    const int Phi = L.Phi;

    int *owner = malloc((size_t)Phi * sizeof(int));
    int64_t *quota = malloc((size_t)Phi * sizeof(int64_t));
    int64_t *rl = calloc((size_t)R, sizeof(int64_t));     /* rank load */
    int *freec = malloc((size_t)R * sizeof(int));
    cand_t *cand = malloc((size_t)Phi * sizeof(cand_t));
    int *ir = malloc((size_t)(R + 1) * sizeof(int));       /* instance ranks  */
    int *is = malloc((size_t)(R + 1) * sizeof(int));       /* instance slots  */
    int64_t *ib = malloc((size_t)(R + 1) * sizeof(int64_t));
    int64_t *iq = malloc((size_t)(R + 1) * sizeof(int64_t));
    int64_t *nq = malloc((size_t)(R + 1) * sizeof(int64_t));

    /* every plan starts from the native placement with all spares free */
    for (int s = 0; s < Phi; s++) {
        owner[s] = L.slot_home[s];
        quota[s] = owner[s] >= 0 ? (int64_t)load[owner[s]] : 0;
        rl[L.slot_rank[s]] += quota[s];
    }
    for (int r = 0; r < R; r++) freec[r] = L.spare_cnt[r];

    int64_t total = 0;
    int bad_load = 0;
    for (int e = 0; e < E; e++) {
        if (load[e] < 0) bad_load = 1;
        total += load[e];
    }
    if (total > INT32_MAX) bad_load = 1;

    const int cap = 2 * L.S + R;
    int steps = 0, cap_hit = 0;
    while (!bad_load) {
        if (steps == cap) { cap_hit = 1; break; }
        /* hottest rank, lowest index on ties */
        int h = 0;
        for (int r = 1; r < R; r++) if (rl[r] > rl[h]) h = r;
        const int64_t old_h = rl[h];

        /* loaded instances on h, by (quota desc, expert asc) */
        int nc = 0;
        for (int s = L.first_slot[h]; s < L.first_slot[h + 1]; s++) {
            if (owner[s] < 0 || quota[s] <= 0) continue;
            cand_t c = { s, owner[s], quota[s] };
            int j = nc++;
            while (j > 0 && (cand[j - 1].quota < c.quota ||
                             (cand[j - 1].quota == c.quota && cand[j - 1].expert > c.expert))) {
                cand[j] = cand[j - 1];
                j--;
            }
            cand[j] = c;
        }
        if (nc == 0) break;

        int committed = 0;
        /* (A) re-level an expert that already has replicas */
        for (int c = 0; c < nc && !committed; c++) {
            int e = cand[c].expert, n = 0, hi = -1;
            for (int s = 0; s < Phi; s++) if (owner[s] == e) {
                ir[n] = L.slot_rank[s]; is[n] = s; iq[n] = quota[s];
                ib[n] = rl[ir[n]] - quota[s];
                if (ir[n] == h) hi = n;
                n++;
            }
            if (n < 2) continue;
            waterfill((int64_t)load[e], n, ib, ir, nq);
            if (ib[hi] + nq[hi] < old_h) {
                for (int i = 0; i < n; i++) { quota[is[i]] = nq[i]; rl[ir[i]] = ib[i] + nq[i]; }
                committed = 1;
            }
        }
        /* (B) replicate onto the least loaded rank with a free spare slot */
        for (int c = 0; c < nc && !committed; c++) {
            int e = cand[c].expert, n = 0, hi = -1;
            for (int s = 0; s < Phi; s++) if (owner[s] == e) {
                ir[n] = L.slot_rank[s]; is[n] = s; iq[n] = quota[s];
                ib[n] = rl[ir[n]] - quota[s];
                if (ir[n] == h) hi = n;
                n++;
            }
            int d = -1;
            const int home_rank = L.slot_rank[L.home_slot[e]];
            for (int r = 0; r < R; r++) {
                if (freec[r] <= 0) continue;
                if (ranks_per_domain > 0 && r / ranks_per_domain != home_rank / ranks_per_domain) continue;
                int hosts = 0;
                for (int i = 0; i < n; i++) if (ir[i] == r) hosts = 1;
                if (hosts) continue;
                if (d < 0 || rl[r] < rl[d]) d = r;
            }
            if (d < 0) continue;
            ir[n] = d; is[n] = L.first_slot[d] + L.nat_cnt[d] + (L.spare_cnt[d] - freec[d]);
            iq[n] = 0; ib[n] = rl[d];
            n++;
            waterfill((int64_t)load[e], n, ib, ir, nq);
            if (ib[hi] + nq[hi] < old_h) {
                owner[is[n - 1]] = e;
                freec[d]--;
                for (int i = 0; i < n; i++) { quota[is[i]] = nq[i]; rl[ir[i]] = ib[i] + nq[i]; }
                committed = 1;
            }
        }
        if (!committed) break;
        steps++;
    }

    /* a replica left without load is released; a native instance never is */
    for (int s = 0; s < Phi; s++)
        if (L.slot_home[s] < 0 && owner[s] >= 0 && quota[s] == 0) owner[s] = -1;

    for (int s = 0; s < Phi; s++) { phy2log[s] = owner[s]; phy_quota[s] = (int32_t)quota[s]; }
    for (int e = 0; e < E; e++) {
        int n = 0;
        for (int s = 0; s < Phi; s++) if (owner[s] == e) {    /* ascending physical slot */
            if (n < rho) log2phy[(int64_t)e * rho + n] = s;
            n++;
        }
        logcnt[e] = n;
        for (int t = n; t < rho; t++) log2phy[(int64_t)e * rho + t] = -1;
    }
    if (steps_out) *steps_out = steps;
    if (cap_hit_out) *cap_hit_out = cap_hit;
    if (bad_load_out) *bad_load_out = bad_load;

    free(owner); free(quota); free(rl); free(freec); free(cand);
    free(ir); free(is); free(ib); free(iq); free(nq);
    layout_free(&L);
    return OR_OK;
}

int or_plan(int32_t E, int32_t R, const int32_t *native_count, const int32_t *native_experts,
            const int32_t *spare_count, const int32_t *load,
            int32_t *phy2log, int32_t *phy_quota, int32_t *logcnt, int32_t *log2phy,
            int32_t rho, int32_t *steps_out, int32_t *cap_hit_out) {
    return or_plan_domain(E, R, native_count, native_experts, spare_count, load, phy2log, phy_quota,
                          logcnt, log2phy, rho, 0, steps_out, cap_hit_out, NULL);
}

/* ------------------------------------------------------------------------- */
/* A3: order-preserving reroute [UltraEP-1: reroute splits the tokens of one */
/* native expert over its replicas; EPLB-5: top-k logical ID -> physical     */
/* replica through the mapping tables].                                      */
/* Returns the number of valid pairs that found no instance (tables whose    */
/* quotas do not cover the load); such pairs get -1, as do padding/invalid.  */
/* ------------------------------------------------------------------------- */
int64_t or_reroute(const int32_t *ids, int64_t n, int32_t E, const int32_t *phy_quota,
                   const int32_t *log2phy, const int32_t *logcnt, int32_t rho, int32_t *phys) {
    int64_t *seen = calloc((size_t)E, sizeof(int64_t));
    int64_t unplaced = 0;
    for (int64_t p = 0; p < n; p++) {
        int32_t v = ids[p];
        if (v < 0 || v >= E) { phys[p] = -1; continue; }
        int64_t j = seen[v]++;
        int64_t acc = 0;
        int32_t out = -1;
        for (int t = 0; t < logcnt[v] && t < rho; t++) {
            int32_t s = log2phy[(int64_t)v * rho + t];
            acc += phy_quota[s];
            if (j < acc) { out = s; break; }
        }
        if (out < 0) unplaced++;
        phys[p] = out;
    }
    free(seen);
    return unplaced;
}

/* ------------------------------------------------------------------------- */
/* A4: gather replica weights into the cross-layer slot buffer [UltraEP-1:   */
/* reserved slots per rank with no runtime allocation; weight buffers reused */
/* across layers].  slot_buf row o belongs to the o-th spare slot in         */
/* rank-major order; empty spare slots are left untouched.                   */
/* ------------------------------------------------------------------------- */
int or_slot_fill(const uint8_t *weights, int64_t bytes_per_expert, int32_t E, int32_t R,
                 const int32_t *native_count, const int32_t *native_experts,
                 const int32_t *spare_count, const int32_t *phy2log, uint8_t *slot_buf) {
    layout_t L;
    int rc = layout_build(&L, E, R, native_count, native_experts, spare_count);
    if (rc != OR_OK) return rc;
    for (int o = 0; o < L.S; o++) {
        int e = phy2log[L.spare_slot[o]];
        if (e < 0 || e >= E) continue; /* not an expert: an empty slot (R15) */
        memcpy(slot_buf + (int64_t)o * bytes_per_expert, weights + (int64_t)e * bytes_per_expert,
               (size_t)bytes_per_expert);
    }
    layout_free(&L);
    return OR_OK;
}

/* ------------------------------------------------------------------------- */
/* A5: balance statistics [UltraEP-4: the most loaded rank relative to the   */
/* average load; EPLB-5: balancedness = mean / max].                         */
/* stats = {max_before, max_after, total, replicas_used};                    */
/* imbalance = {before, after} = max * R / total (1.0 when total == 0).     */
/* ------------------------------------------------------------------------- */
int or_stats(int32_t E, int32_t R, const int32_t *native_count, const int32_t *native_experts,
             const int32_t *spare_count, const int32_t *load, const int32_t *phy_quota,
             int64_t *stats, int32_t *rank_load, double *imbalance) {
    layout_t L;
    int rc = layout_build(&L, E, R, native_count, native_experts, spare_count);
    if (rc != OR_OK) return rc;
    int64_t max_b = 0, max_a = 0, total = 0, used = 0;
    for (int r = 0; r < R; r++) {
        int64_t before = 0, after = 0;
        for (int s = L.first_slot[r]; s < L.first_slot[r + 1]; s++) {
            if (L.slot_home[s] >= 0) before += load[L.slot_home[s]];
            else if (phy_quota[s] > 0) used++;
            after += phy_quota[s];
        }
        if (rank_load) { rank_load[r] = (int32_t)before; rank_load[R + r] = (int32_t)after; }
        if (before > max_b) max_b = before;
        if (after > max_a) max_a = after;
    }
    for (int e = 0; e < E; e++) total += load[e];
    stats[0] = max_b; stats[1] = max_a; stats[2] = total; stats[3] = used;
    imbalance[0] = total > 0 ? (double)(max_b * (int64_t)R) / (double)total : 1.0;
    imbalance[1] = total > 0 ? (double)(max_a * (int64_t)R) / (double)total : 1.0;
    layout_free(&L);
    return OR_OK;
}

/* Physical slot numbering, exposed so tests can check it independently. */
int or_layout(int32_t E, int32_t R, const int32_t *native_count, const int32_t *native_experts,
              const int32_t *spare_count, int32_t *first_slot, int32_t *slot_home,
              int32_t *slot_rank, int32_t *spare_slot) {
    layout_t L;
    int rc = layout_build(&L, E, R, native_count, native_experts, spare_count);
    if (rc != OR_OK) return rc;
    for (int r = 0; r <= R; r++) first_slot[r] = L.first_slot[r];
    for (int s = 0; s < L.Phi; s++) { slot_home[s] = L.slot_home[s]; slot_rank[s] = L.slot_rank[s]; }
    for (int o = 0; o < L.S; o++) spare_slot[o] = L.spare_slot[o];
    layout_free(&L);
    return OR_OK;
}

/* Water-filling on its own, for the closed-form pins. */
int or_waterfill(int64_t T, int32_t n, const int64_t *b, const int32_t *rank, int64_t *q) {
    int *rk = malloc((size_t)(n > 0 ? n : 1) * sizeof(int));
    for (int i = 0; i < n; i++) rk[i] = rank[i];
    waterfill(T, n, b, rk, q);
    free(rk);
    return OR_OK;
}

/* ------------------------------------------------------------------------- */
/* Next row: dispatch layout for the token all-to-all [EPLB tutorial, EPLB / */
/* DeepEP section: dispatch sends each pair to its physical replica, combine */
/* gathers the results back to the logical expert].  Pairs are laid out     */
/* physical-slot-major: slot s owns positions [off_s, off_s + quota_s) with   */
/* off the exclusive prefix of the quotas in slot order, and the j-th pair of */
/* expert e, served by instance s whose range starts at Q, sits at           */
/* off_s + (j - Q).  pos[p] is that position (-1 for padding, invalid IDs    */
/* and pairs past the expert's quotas); src[k] is the pair at position k     */
/* (-1 where no pair lands).  Returns the number of placed pairs.            */
/* ------------------------------------------------------------------------- */
int64_t or_dispatch(const int32_t *ids, int64_t n, int32_t E, int32_t Phi, const int32_t *phy_quota,
                    const int32_t *log2phy, const int32_t *logcnt, int32_t rho,
                    int64_t *slot_off, int32_t *pos, int32_t *src) {
    slot_off[0] = 0;
    for (int s = 0; s < Phi; s++) slot_off[s + 1] = slot_off[s] + phy_quota[s];
    for (int64_t k = 0; k < n; k++) src[k] = -1;
    int64_t *seen = calloc((size_t)E, sizeof(int64_t));
    int64_t placed = 0;
    for (int64_t p = 0; p < n; p++) {
        int32_t v = ids[p];
        pos[p] = -1;
        if (v < 0 || v >= E) continue;
        int64_t j = seen[v]++;
        int64_t Q = 0;
        for (int t = 0; t < logcnt[v] && t < rho; t++) {
            int32_t s = log2phy[(int64_t)v * rho + t];
            if (j < Q + phy_quota[s]) {
                int64_t k = slot_off[s] + (j - Q);
                pos[p] = (int32_t)k;
                if (k < n) src[k] = (int32_t)p;
                placed++;
                break;
            }
            Q += phy_quota[s];
        }
    }
    free(seen);
    return placed;
}

/* ------------------------------------------------------------------------- */
/* Next row: replica gradient reduction [UltraEP article, key designs:       */
/* replicas keep no optimizer state and their gradients are reduced back to  */
/* the native expert during backward; the backward paragraph: accumulation   */
/* keeps a fixed order so the reduction is deterministic].  For every expert */
/* with replicas, its gradient becomes the fp32 fold of its instances'       */
/* gradients in ascending physical-slot order:                               */
/*     acc = g(inst 0); acc = acc + g(inst 1); ...                            */
/* where the native instance reads native_grads[e] and a replica in spare    */
/* slot o reads slot_grads[o].  The result overwrites native_grads[e].       */
/* ------------------------------------------------------------------------- */
int or_grad_reduce(float *native_grads, int64_t n, const float *slot_grads, int32_t E, int32_t R,
                   const int32_t *native_count, const int32_t *native_experts,
                   const int32_t *spare_count, const int32_t *log2phy, const int32_t *logcnt,
                   int32_t rho) {
    layout_t L;
    int rc = layout_build(&L, E, R, native_count, native_experts, spare_count);
    if (rc != OR_OK) return rc;
    int *spare_of = malloc((size_t)L.Phi * sizeof(int));
    for (int s = 0; s < L.Phi; s++) spare_of[s] = -1;
    for (int o = 0; o < L.S; o++) spare_of[L.spare_slot[o]] = o;
    for (int e = 0; e < E; e++) {
        int c = logcnt[e] < rho ? logcnt[e] : rho;
        if (c < 2) continue;
        const float **rows = malloc((size_t)c * sizeof(float *));
        for (int t = 0; t < c; t++) {
            int s = log2phy[(int64_t)e * rho + t];
            rows[t] = L.slot_home[s] >= 0 ? native_grads + (int64_t)L.slot_home[s] * n
                                          : slot_grads + (int64_t)spare_of[s] * n;
        }
        float *out = native_grads + (int64_t)e * n;
        for (int64_t k = 0; k < n; k++) {
            float acc = rows[0][k];
            for (int t = 1; t < c; t++) acc = acc + rows[t][k];
            out[k] = acc;
        }
        free(rows);
    }
    free(spare_of);
    layout_free(&L);
    return OR_OK;
}
