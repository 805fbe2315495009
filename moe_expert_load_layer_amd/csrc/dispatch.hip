// Dispatch layout for the token all-to-all (EPLB tutorial, EPLB / DeepEP
// section: dispatch sends each pair to its physical replica, combine gathers
// the results back to the logical expert).  The pairs of a plan are laid out
// physical-slot-major: slot s owns positions [off_s, off_s + quota_s), off
// the exclusive prefix of the quotas in slot order, and the j-th pair of
// expert e, served by instance s whose quota range starts at Q, goes to
// position off_s + (j - Q).  With quotas that cover the loads this is the
// stable counting sort of the pairs by physical slot.
//
// One wave per sub-block (the histogram's); each workgroup builds the plan's
// route table (slot offsets, per-instance (end, off - Q)) once and its waves
// then walk one or more sub-blocks (see the launcher).  Every pair needs its rank among the pairs of
// its expert, so each 64-pair column is ranked with an LDS bit mask per
// expert (each lane ORs its bit, counts the bits below it) plus a per-expert
// running count; the first rank of the expert in the sub-block comes from the
// histogram's workspace rows.  Positions are unique, so the writes of
// dispatch_src never collide.
//
// dispatch_src is written through LDS when the staging buffer leaves enough
// waves resident: each wave stages the in-sub-block index of every pair at
// (its cell's offset + its rank), marks where each non-empty cell starts, and
// then writes the staged slots in order, 64 at a time; a cell's pairs go to
// consecutive positions, so each store writes a few coalesced runs.
// Otherwise each pair's index is stored at its position directly, and the
// launch runs plan by plan so that those scattered stores meet in the caches.
#include <type_traits>

#include "ep_internal.h"

namespace ep {
namespace {

// Per-expert state of a wave's sub-block (16 bytes): the bit mask of the
// current 64-pair column, the count of the expert's pairs in earlier columns
// with two flags in its top bits, and the position base: run + (off - Q) of
// the one instance that takes all of the expert's pairs here, or the run
// itself when a quota boundary falls inside (split), so that the k-th pair
// of the cell goes to base + k, or to the instance a search of run + k finds.
struct Cell1 {
    uint64_t mask;
    uint32_t kf;
    int32_t base;
};
// ranking two columns per LDS round trip keeps a mask per column
struct Cell2 {
    uint64_t mask;   // lanes of the first column of the current pair
    uint64_t mask1;  // lanes of the second column
    uint32_t kf;
    int32_t base;
};
template <bool PAIR> using CellOf = typename std::conditional<PAIR, Cell2, Cell1>::type;
template <bool PAIR> __device__ __forceinline__ CellOf<PAIR> make_cell(uint32_t kf, int32_t base) {
    CellOf<PAIR> c;
    c.mask = 0ull;
    if constexpr (PAIR) c.mask1 = 0ull;
    c.kf = kf;
    c.base = base;
    return c;
}
constexpr uint32_t kSplitFlag = 1u << 30;  // a quota boundary falls inside the cell
constexpr uint32_t kNoneFlag = 1u << 31;   // no instance takes these pairs
constexpr uint32_t kCountMask = kSplitFlag - 1;

__device__ __forceinline__ int32_t position_of(const int2 *inst, int f, int n, int32_t j) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (j < inst[f + mid].x) hi = mid; else lo = mid + 1;
    }
    if (lo < n && inst[f + lo].y != (int32_t)0x80000000) return j + inst[f + lo].y;
    return -1;
}

template <int W, bool STAGED, bool PAIR>
__global__ __launch_bounds__(W *kWave) void dispatch_kernel(
    const int32_t *__restrict__ ids, int64_t N, int32_t E, int32_t Phi, int32_t rho, int64_t sub,
    int64_t nsb, int64_t sps, int64_t nseg, const int32_t *__restrict__ ws, const int32_t *__restrict__ phy_quota,
    const int32_t *__restrict__ log2phy, const int32_t *__restrict__ logcnt,
    int32_t *__restrict__ slot_offsets, int32_t *__restrict__ dpos, int32_t *__restrict__ dsrc) {
    extern __shared__ __align__(16) unsigned char sh_raw[];
    const int64_t nwords = STAGED ? sub / kWave : 0;                         // cell-start bit words
    const int E1c = E + 1;                                                  // cell E: padding, bad IDs
    const int64_t sstride = STAGED ? sub + kWave : 0;                       // slot sub: sink
    using Cell = CellOf<PAIR>;
    Cell *cell_all = reinterpret_cast<Cell *>(sh_raw);                      // [W][E+1]
    uint64_t *sbits_all = reinterpret_cast<uint64_t *>(cell_all + (size_t)W * E1c); // [W][sub/64] if STAGED
    int2 *inst = reinterpret_cast<int2 *>(sbits_all + (size_t)W * nwords);  // [Phi] (end, off - Q)
    int32_t *soff = reinterpret_cast<int32_t *>(inst + Phi);                // [Phi + 1]
    int32_t *rfirst = soff + Phi + 1;                                       // [E]
    int32_t *rcnt = rfirst + E;                                             // [E]
    int32_t *nel_all = rcnt + E;                                            // [W][E] if STAGED
    int32_t *off_all = nel_all + (STAGED ? (size_t)W * E : 0);              // [W][E] if STAGED
    uint16_t *stage_all = reinterpret_cast<uint16_t *>(off_all + (STAGED ? (size_t)W * E : 0)); // [W][sub + 64]
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int p = blockIdx.y;
    const int E1 = E + 1;

    if (wave == 0) {
        // slot offsets: exclusive prefix of the quotas in slot order
        int carry = 0;
        for (int c = 0; c < Phi; c += kWave) {
            const int s = c + lane;
            const int q = s < Phi ? phy_quota[(int64_t)p * Phi + s] : 0;
            const int incl = wave_incl_scan_i32(q);
            if (s < Phi) soff[s] = carry + incl - q;
            carry += __shfl(incl, kWave - 1);
        }
        if (lane == 0) soff[Phi] = carry;
        // instance lists of the experts
        carry = 0;
        for (int c = 0; c < E; c += kWave) {
            const int e = c + lane;
            int n = 0;
            if (e < E) {
                n = logcnt[(int64_t)p * E + e];
                n = n < 0 ? 0 : (n > rho ? rho : n);
            }
            const int incl = wave_incl_scan_i32(n);
            if (e < E) {
                int start = carry + incl - n;
                if (start > Phi) start = Phi;
                if (start + n > Phi) n = Phi - start;
                rfirst[e] = start;
                rcnt[e] = n;
            }
            carry += __shfl(incl, kWave - 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += W * kWave) {
        const int f = rfirst[e], n = rcnt[e];
        const int32_t *row = log2phy + ((int64_t)p * E + e) * rho;
        int32_t acc = 0;
        for (int t = 0; t < n; t++) {
            const int s = row[t];
            const bool ok = s >= 0 && s < Phi;
            const int32_t q = ok ? phy_quota[(int64_t)p * Phi + s] : 0;
            inst[f + t] = make_int2(acc + q, ok ? soff[s] - acc : 0x80000000);
            acc += q;
        }
    }
    if (blockIdx.x == 0) {
        for (int s = threadIdx.x; s <= Phi; s += W * kWave) slot_offsets[(int64_t)p * (Phi + 1) + s] = soff[s];
        // an instance whose quota range reaches past its expert's load (a plan
        // whose quotas exceed the loads) leaves positions no pair takes: they
        // get -1 here (none for plans whose quotas equal the loads); the pairs'
        // own positions and the tail past the total are written below
        const int32_t *tot = ws + ((int64_t)p * (nsb + nseg + 1) + nsb + nseg) * E1;
        int32_t *srow = dsrc + (int64_t)p * N;
        for (int e = threadIdx.x; e < E; e += W * kWave) {
            const int f = rfirst[e], n = rcnt[e];
            const int32_t le = tot[e];
            int32_t prev = 0;
            for (int t = 0; t < n; t++) {
                const int2 in = inst[f + t];
                if (in.y != (int32_t)0x80000000)
                    for (int64_t j = prev > le ? prev : le; j < in.x; j++) {
                        const int64_t pos = j + in.y;
                        if (pos >= 0 && pos < N) srow[pos] = -1;
                    }
                prev = in.x;
            }
        }
    }
    __syncthreads();

    // each wave walks the plan's sub-blocks with a stride of the plan's waves,
    // reusing the block's route table; no block barriers below
    for (int64_t sb = (int64_t)blockIdx.x * W + wave; sb < nsb; sb += (int64_t)gridDim.x * W) {
    wave_lds_fence();  // the previous sub-block's reads of the wave's LDS are done
    Cell *cells = cell_all + (size_t)wave * E1c;
    int32_t *offs = off_all + (size_t)wave * (STAGED ? E : 0);  // staging offset of each cell
    uint16_t *stage = stage_all + (size_t)wave * sstride;
    uint64_t *sbits = sbits_all + (size_t)wave * nwords;   // bit t: staged slot t starts a cell
    int32_t *nel = nel_all + (size_t)wave * (STAGED ? E : 0);  // non-empty cells' experts, in order
    const SubPrefix pre = sub_prefix(ws, p, sb, nsb, sps, nseg, E1);
    int staged_pairs = 0;
    if (STAGED) {
        for (int64_t w = lane; w < nwords; w += kWave) sbits[w] = 0ull;
        wave_lds_fence();
    }
    {
        int carry = 0, ncells = 0;
        for (int c = 0; c < E; c += kWave) {
            const int e = c + lane;
            int32_t run = 0, cnt = 0, base = 0;
            uint32_t flags = kNoneFlag;
            if (e < E) {
                run = pre.start(e);
                cnt = pre.end(e) - run;
                const int f = rfirst[e], n = rcnt[e];
                int lo = 0, hi = n;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (run < inst[f + mid].x) hi = mid; else lo = mid + 1;
                }
                base = run;
                if (cnt > 0 && lo < n && inst[f + lo].y != (int32_t)0x80000000) {
                    if (run + cnt <= inst[f + lo].x) {
                        flags = 0;
                        base = run + inst[f + lo].y;
                    } else {
                        flags = kSplitFlag;
                    }
                } else if (cnt > 0 && lo < n) {
                    flags = kSplitFlag;
                }
            }
            const int incl = wave_incl_scan_i32(cnt);
            const int off = carry + incl - cnt;
            if (e < E) {
                cells[e] = make_cell<PAIR>(flags, base);
                if (STAGED) offs[e] = off;
            }
            if (STAGED) {
                const bool full = e < E && cnt > 0;
                const uint64_t fm = __ballot(full);
                if (full) {
                    nel[ncells + __popcll(fm & lanemask_lt())] = e;
                    atomicOr(reinterpret_cast<unsigned long long *>(&sbits[off / kWave]),
                             1ull << (off % kWave));
                }
                ncells += __popcll(fm);
            }
            carry += __shfl(incl, kWave - 1);
        }
        staged_pairs = carry;
        if (lane == 0) cells[E] = make_cell<PAIR>(kNoneFlag, 0);
    }
    wave_lds_fence();

    const int64_t begin = sb * sub;
    const int64_t end = (begin + sub < N) ? begin + sub : N;
    const int32_t *src = ids + (int64_t)p * N;
    int32_t *pos_out = dpos + (int64_t)p * N;
    int32_t *src_out = dsrc + (int64_t)p * N;
    const uint64_t lt = lanemask_lt();
    const uint64_t bit = 1ull << lane;
    const uint32_t uE = (uint32_t)E;
    constexpr int U = 8;
    // the IDs of the next U columns load while the current ones are ranked
    // (the loads are unconditional, from a clamped index, so that the wait
    // for a group's IDs does not also wait for the next group's)
    const int64_t last = end - 1;
    int32_t nxt[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int64_t i = begin + u * kWave + lane;
        const int32_t t = __builtin_nontemporal_load(src + (i < end ? i : last));
        nxt[u] = i < end ? t : -1;
    }
    // whole groups of U columns store every pair's position unconditionally:
    // a store under a branch leaves the compiler unable to count the stores
    // issued after the prefetched ID loads, and its wait for those loads then
    // also waits for every store (stores and loads share one counter here)
    auto group = [&](int64_t g, auto fullc) {
        constexpr bool FULL = decltype(fullc)::value;
        int32_t v[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            v[u] = nxt[u];
            const int64_t i = g + (U + u) * kWave + lane;
            const int32_t t = __builtin_nontemporal_load(src + (i < end ? i : last));
            nxt[u] = i < end ? t : -1;
        }
        if constexpr (PAIR) {
            // two columns per LDS round trip: each ORs its lanes into its own
            // mask of the expert's cell, one read then ranks both (a pair in the
            // second column also counts all of its expert's pairs in the first),
            // and the expert's first lane in the pair folds both masks into the
            // count
            static_assert(U % 2 == 0, "columns go in pairs");
    #pragma unroll
            for (int u = 0; u < U; u += 2) {
                const int32_t xa = v[u], xb = v[u + 1];
                const bool va = (uint32_t)xa < uE, vb = (uint32_t)xb < uE;
                const int ia = va ? xa : E, ib = vb ? xb : E;  // padding and bad IDs rank in the sink cell
                atomicOr(reinterpret_cast<unsigned long long *>(&cells[ia].mask), bit);
                atomicOr(reinterpret_cast<unsigned long long *>(&cells[ib].mask1), bit);
                wave_lds_fence();
                const Cell ca = cells[ia];
                const Cell cb = cells[ib];
                const int32_t offa = STAGED && va ? offs[ia] : 0;
                const int32_t offb = STAGED && vb ? offs[ib] : 0;
                wave_lds_fence();
                const uint64_t belowa = ca.mask & lt;
                const uint64_t belowb = cb.mask1 & lt;
                // one lane per expert of the pair: its lowest in the first column,
                // else (absent there) its lowest in the second
                if (belowa == 0)
                    cells[ia] = make_cell<PAIR>(ca.kf + (uint32_t)__popcll(ca.mask) + (uint32_t)__popcll(ca.mask1), ca.base);
                if (cb.mask == 0 && belowb == 0)
                    cells[ib] = make_cell<PAIR>(cb.kf + (uint32_t)__popcll(cb.mask1), cb.base);
                const int32_t ka = (int32_t)(ca.kf & kCountMask) + (int32_t)__popcll(belowa);
                const int32_t kb = (int32_t)(cb.kf & kCountMask) + (int32_t)__popcll(cb.mask) + (int32_t)__popcll(belowb);
                auto place = [&](const Cell &c, int xi, bool valid, int32_t off, int32_t k, int64_t i) {
                    int32_t pos = (c.kf & (kNoneFlag | kSplitFlag)) ? -1 : c.base + k;
                    if (c.kf & kSplitFlag) pos = position_of(inst, rfirst[xi], rcnt[xi], c.base + k);
                    if (STAGED) stage[valid ? off + k : sub] = (uint16_t)(i - begin);
                    else if (pos >= 0 && pos < N) src_out[pos] = (int32_t)i;
                    if (FULL || i < end) __builtin_nontemporal_store(pos, pos_out + i);
                };
                place(ca, ia, va, offa, ka, g + u * kWave + lane);
                place(cb, ib, vb, offb, kb, g + (u + 1) * kWave + lane);
                wave_lds_fence();
            }
    
        } else {
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int32_t x = v[u];
                const bool valid = (uint32_t)x < uE;
                const int xi = valid ? x : E;  // padding and bad IDs rank in the sink cell
                atomicOr(reinterpret_cast<unsigned long long *>(&cells[xi].mask), bit);
                wave_lds_fence();
                const Cell cur = cells[xi];
                const int32_t off = STAGED && valid ? offs[xi] : 0;
                wave_lds_fence();
                const int64_t i = g + u * kWave + lane;
                const uint64_t below = cur.mask & lt;
                if (below == 0) cells[xi] = make_cell<PAIR>(cur.kf + (uint32_t)__popcll(cur.mask), cur.base);
                const int32_t k = (int32_t)(cur.kf & kCountMask) + (int32_t)__popcll(below);
                int32_t pos = (cur.kf & (kNoneFlag | kSplitFlag)) ? -1 : cur.base + k;
                if (cur.kf & kSplitFlag) pos = position_of(inst, rfirst[xi], rcnt[xi], cur.base + k);
                if (STAGED) stage[valid ? off + k : sub] = (uint16_t)(i - begin);
                else if (pos >= 0 && pos < N) src_out[pos] = (int32_t)i;
                if (FULL || i < end) __builtin_nontemporal_store(pos, pos_out + i);
                wave_lds_fence();
            }
        }
    };
    // (only in the staged form: the non-staged one stores dispatch_src under a
    // branch anyway, and the second copy of the loop costs it registers and
    // resident waves: 7 % slower on the stress batch)
    {
        int64_t g = begin;
        if constexpr (STAGED)
            for (; g + U * kWave <= end; g += U * kWave) group(g, std::true_type{});
        for (; g < end; g += U * kWave) group(g, std::false_type{});
    }
    if (STAGED) {
        // staged slots in order, 64 per step: slot t belongs to the non-empty
        // cell whose start is the last one at or before t; each expert's
        // slots go to consecutive positions (per instance), so every store
        // writes a few coalesced runs
        constexpr int UF = 4;  // windows per step: their LDS reads overlap
        const uint64_t upto = lane == kWave - 1 ? ~0ull : ((2ull << lane) - 1);
        int cbase = -1;  // cells started before the current window, minus one
        for (int w0 = 0; w0 < staged_pairs; w0 += UF * kWave) {
            uint64_t word[UF];
            int cb[UF];
#pragma unroll
            for (int u = 0; u < UF; u++) {
                const int64_t wi = w0 / kWave + u;
                word[u] = wi < nwords ? sbits[wi] : 0ull;
            }
#pragma unroll
            for (int u = 0; u < UF; u++) {
                cb[u] = cbase;
                cbase += __popcll(word[u]);
            }
            int e[UF];
            uint16_t sidx[UF];
#pragma unroll
            for (int u = 0; u < UF; u++) {
                const int t = w0 + u * kWave + lane;
                e[u] = t < staged_pairs ? nel[cb[u] + __popcll(word[u] & upto)] : 0;
                sidx[u] = t < staged_pairs ? stage[t] : 0;
            }
#pragma unroll
            for (int u = 0; u < UF; u++) {
                const int t = w0 + u * kWave + lane;
                if (t < staged_pairs) {
                    const Cell cell = cells[e[u]];
                    const int32_t k = t - offs[e[u]];
                    int32_t pos = -1;
                    if (cell.kf & kSplitFlag) pos = position_of(inst, rfirst[e[u]], rcnt[e[u]], cell.base + k);
                    else if (!(cell.kf & kNoneFlag)) pos = cell.base + k;
                    if (pos >= 0 && pos < N) src_out[pos] = (int32_t)(begin + sidx[u]);
                }
            }
        }
    }
    // positions past the plan's total quota hold no pair
    const int64_t tail = soff[Phi] > begin ? soff[Phi] : begin;
    for (int64_t i = tail + lane; i < end; i += kWave) src_out[i] = -1;
    }
}

int pick_dispatch_waves(int E, int Phi, int64_t stage, bool pair) {
    for (int w = 4; w >= 1; w >>= 1)
        if (dispatch_lds_bytes(E, Phi, w, stage, pair) <= kLdsPreferred) return w;
    return dispatch_lds_bytes(E, Phi, 1, stage, pair) <= kLdsMax ? 1 : 0;
}

}  // namespace

size_t dispatch_lds_bytes(int E, int Phi, int waves, int64_t stage_pairs, bool pair) {
    const size_t staged = stage_pairs > 0 ? (size_t)waves * ((size_t)stage_pairs / kWave * 8 + (size_t)E * 8 +
                                                             ((size_t)stage_pairs + kWave) * 2)
                                          : 0;
    return (size_t)waves * (E + 1) * (pair ? sizeof(Cell2) : sizeof(Cell1)) + (size_t)Phi * 8 +
           (size_t)(Phi + 1) * 4 + (size_t)E * 8 + staged;
}

template <bool ST, bool PR>
static const void *dispatch_fn_w(int w) {
    return w == 4 ? (const void *)dispatch_kernel<4, ST, PR>
                  : w == 2 ? (const void *)dispatch_kernel<2, ST, PR> : (const void *)dispatch_kernel<1, ST, PR>;
}

static const void *dispatch_fn(int w, bool staged, bool pair) {
    if (staged) return pair ? dispatch_fn_w<true, true>(w) : dispatch_fn_w<true, false>(w);
    return pair ? dispatch_fn_w<false, true>(w) : dispatch_fn_w<false, false>(w);
}

static int resident_blocks(int w, bool staged, bool pair, size_t lds) {
    return ::ep::resident_blocks(dispatch_fn(w, staged, pair), w * kWave, lds);
}

hipError_t launch_dispatch(const int32_t *ids, int64_t N, int32_t P, const ep_layout_t &L,
                           const SubGeom &g, const int32_t *ws, const int32_t *phy_quota,
                           const int32_t *log2phy, const int32_t *logcnt, int32_t *slot_offsets,
                           int32_t *dpos, int32_t *dsrc, hipStream_t s) {
    const int64_t sub = g.sub, nsb = g.nsb, sps = g.sps, nseg = g.nseg;
    const int E = L.num_experts, Phi = L.num_phys, rho = L.max_replicas;
    // stage through LDS when a sub-block's pair indices fit (16-bit); of the
    // wave counts whose LDS fits a workgroup, take the one with the most
    // resident waves (the kernel is bound by LDS latency, so occupancy counts)
    // Staging turns the scatter of dispatch_src into runs, but its buffer
    // (2 bytes per pair of a sub-block) lowers occupancy; below 8 resident
    // waves per CU the direct scatter is faster.
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        cus = 0;
    }
    // Ranking two columns per LDS round trip pays where a few hot experts fill
    // the columns (GLM-4.5-like and stress batches 25 % and 8 % faster), but its
    // larger cells cost the 128-expert layout resident waves (17 % slower); so
    // pairs above 128 experts, when their cells fit in LDS.
    const bool pair = E > 128 && dispatch_lds_bytes(E, Phi, 1, 0, true) <= kLdsPreferred;
    auto best_waves = [&](bool st, int &w_out) {
        const int w0 = pick_dispatch_waves(E, Phi, st ? sub : 0, pair);
        int best = w0, waves = -1;
        for (int c = w0; c >= 1; c >>= 1) {
            const int r = resident_blocks(c, st, pair, dispatch_lds_bytes(E, Phi, c, st ? sub : 0, pair));
            if (r * c > waves) { best = c; waves = r * c; }
        }
        w_out = w0 > 0 ? best : 0;
        return w0 > 0 ? waves : -1;
    };
    int w = 0, wu = 0;
    const int ws_waves = sub <= 65536 ? best_waves(true, w) : -1;
    bool staged = ws_waves >= 0 && w > 0;
    if (!staged || (cus > 0 && ws_waves < 8 * cus)) {
        const int wu_waves = best_waves(false, wu);
        if (wu > 0 && (!staged || wu_waves > ws_waves)) { staged = false; w = wu; }
    }
    if (w == 0) return hipErrorInvalidValue;
    const size_t lds = dispatch_lds_bytes(E, Phi, w, staged ? sub : 0, pair);
    // Blocks per plan.  Staged: every block builds the plan's route table once,
    // so a launch of many plans uses no more blocks than the GPU holds at once
    // (one round, equal work), each wave walking many sub-blocks.  Direct: one
    // sub-block per wave; workgroups are dispatched x-fastest, so plan by plan,
    // and the scattered 4-byte dispatch_src stores of the few plans in flight
    // merge in the caches before they reach HBM (with every plan in flight they
    // do not: stress batch 7.4 -> 6.4 ms).  At least one block per plan, so the
    // slot offsets are always written.
    int64_t nblk = nsb > 0 ? (nsb + w - 1) / w : 1;
    const int resident = resident_blocks(w, staged, pair, lds);
    if (staged && resident > 0) {
        const int64_t per_plan = resident / P > 0 ? resident / P : 1;
        if (per_plan < nblk) nblk = per_plan;
    }
    dim3 grid((unsigned)nblk, (unsigned)P);
#define EP_DISPATCH(WV, ST, PR)                                                                         \
    hipLaunchKernelGGL((dispatch_kernel<WV, ST, PR>), grid, dim3(WV * kWave), lds, s, ids, N, E, Phi, rho, \
                       sub, nsb, sps, nseg, ws, phy_quota, log2phy, logcnt, slot_offsets, dpos, dsrc)
#define EP_DISPATCH_W(ST, PR)                                                                           \
    do {                                                                                                \
        if (w == 4) EP_DISPATCH(4, ST, PR); else if (w == 2) EP_DISPATCH(2, ST, PR); else EP_DISPATCH(1, ST, PR); \
    } while (0)
    if (staged) {
        if (pair) EP_DISPATCH_W(true, true); else EP_DISPATCH_W(true, false);
    } else {
        if (pair) EP_DISPATCH_W(false, true); else EP_DISPATCH_W(false, false);
    }
#undef EP_DISPATCH_W
#undef EP_DISPATCH
    return hipGetLastError();
}

}  // namespace ep
