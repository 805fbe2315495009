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
// then walk one or more sub-blocks (see the launcher).  Every pair needs its
// rank among the pairs of its expert, so each 64-pair column is ranked with an
// LDS bit mask per expert (each lane ORs its bit, counts the bits below it)
// plus a per-expert running count; the first rank of the expert in the
// sub-block comes from the histogram's workspace rows.  Positions are unique, so the writes of
// dispatch_src never collide.
//
// dispatch_src is written through LDS when the staging buffer leaves enough
// waves resident: each wave stages the in-sub-block index of every pair at
// (its cell's offset + its rank), marks where each non-empty cell ends, and
// then writes the staged slots in order, 64 at a time; a cell's pairs go to
// consecutive positions, so each store writes a few coalesced runs.
// Otherwise each pair's index is stored at its position directly, and the
// launch runs plan by plan so that those scattered stores meet in the caches.
#include <type_traits>

#include "ep_internal.h"

namespace ep {
namespace {

// Per-expert state of a wave's sub-block (a "cell"): the bit mask of the
// current 64-pair column; kf, the cell's staging offset plus the count of the
// expert's pairs in earlier columns, with two flags in its top bits; and
// base, the position base plus that count: the base is run + (off - Q) of the
// one instance that takes all of the expert's pairs here, or the run itself
// when a quota boundary falls inside (split), so that the k-th pair of the
// cell goes to base + k, or to the instance a search of run + k finds, and is
// staged at off + k.
// In LDS the fields live in separate arrays over the experts (masks, then
// (count, base) pairs): the column's 8-byte mask accesses of neighbouring
// experts then fall in neighbouring banks (with 16-byte cells the
// Qwen3-like batch took 1.8 times the bank-conflict cycles, and the staged
// batches ran 2-8 % slower).  These structs hold one cell's values in
// registers.
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
    // a wave's cells: column masks [E+1] (two arrays if PAIR), then (count
    // with flags, base) [E+1]
    constexpr int kCellWords = PAIR ? 3 : 2;
    uint64_t *cell_all = reinterpret_cast<uint64_t *>(sh_raw);              // [W][kCellWords][E+1]
    uint64_t *sbits_all = cell_all + (size_t)W * kCellWords * E1c;           // [W][sub/64] if STAGED
    int2 *inst = reinterpret_cast<int2 *>(sbits_all + (size_t)W * nwords);  // [Phi] (end, off - Q)
    int32_t *soff = reinterpret_cast<int32_t *>(inst + Phi);                // [Phi + 1]
    int32_t *rfirst = soff + Phi + 1;                                       // [E]
    int32_t *rcnt = rfirst + E;                                             // [E]
    // [W][E+1] if STAGED: per non-empty cell, in order, what the flush needs:
    // (position - staged slot, 0), (run - staging offset, expert | split) or
    // (0, none); aligned by an offset from the LDS base (an integer round
    // trip of the pointer would lose its address space and turn every access
    // into a flat one)
    int2 *cinfo_all = reinterpret_cast<int2 *>(
        sh_raw + ((reinterpret_cast<unsigned char *>(rcnt + E) - sh_raw + 7) & ~(ptrdiff_t)7));
    uint16_t *stage_all = reinterpret_cast<uint16_t *>(cinfo_all + (STAGED ? (size_t)W * (E + 1) : 0)); // [W][sub + 64]
    // (the wave index is uniform in a wave: read into a scalar register, so
    // that the sub-block loop, its bounds and bases stay scalar)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
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
    // workgroups go to the 8 XCDs round-robin: the ones on one XCD take
    // consecutive sub-blocks, so that the runs of neighbouring sub-blocks in
    // dispatch_src meet in one L2
    int64_t lblk;
    {
        const int nb = (int)gridDim.x, x = (int)blockIdx.x;
        const int q = nb / 8, r = nb % 8, c = x % 8, j = x / 8;
        lblk = c < r ? (int64_t)c * (q + 1) + j : (int64_t)r * (q + 1) + (int64_t)(c - r) * q + j;
    }
    for (int64_t sb = lblk * W + wave; sb < nsb; sb += (int64_t)gridDim.x * W) {
    wave_lds_fence();  // the previous sub-block's reads of the wave's LDS are done
    uint64_t *mk0 = cell_all + (size_t)wave * kCellWords * E1c;
    uint64_t *mk1 = mk0 + E1c;  // PAIR only
    uint2 *inf = reinterpret_cast<uint2 *>(mk0 + (size_t)(kCellWords - 1) * E1c);
    uint16_t *stage = stage_all + (size_t)wave * sstride;
    uint64_t *sbits = sbits_all + (size_t)wave * nwords;   // bit t: staged slot t ends a cell
    int2 *cinfo = cinfo_all + (size_t)wave * (STAGED ? E + 1 : 0);
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
                mk0[e] = 0ull;
                if (PAIR) mk1[e] = 0ull;
                inf[e] = make_uint2((STAGED ? (uint32_t)off : 0u) | flags, (uint32_t)base);
            }
            if (STAGED) {
                const bool full = e < E && cnt > 0;
                const uint64_t fm = __ballot(full);
                if (full) {
                    int2 ci = make_int2(base - off, 0);
                    if (flags & kNoneFlag) ci = make_int2(0, (int32_t)kNoneFlag);
                    else if (flags & kSplitFlag) ci = make_int2(base - off, e | (int32_t)kSplitFlag);
                    cinfo[ncells + __popcll(fm & lanemask_lt())] = ci;
                    const int last = off + cnt - 1;
                    atomicOr(reinterpret_cast<unsigned long long *>(&sbits[last / kWave]),
                             1ull << (last % kWave));
                }
                ncells += __popcll(fm);
            }
            carry += __shfl(incl, kWave - 1);
        }
        // (uniform: the flush loop below then runs on scalar registers)
        staged_pairs = __builtin_amdgcn_readfirstlane(carry);
        if (STAGED && lane == 0) cinfo[ncells] = make_int2(0, (int32_t)kNoneFlag);  // read by slots past the staged pairs
        if (lane == 0) {
            mk0[E] = 0ull;
            if (PAIR) mk1[E] = 0ull;
            inf[E] = make_uint2(kNoneFlag, 0u);
        }
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
    // pair offsets within the sub-block are 32-bit (a sub-block is far below
    // 2^30 pairs), so the loads and the position stores address from a
    // scalar base plus a 32-bit byte offset (with 64-bit indices the kernel
    // issued 6 % more vector instructions and held 120 instead of 71
    // registers)
    const char *srcb = reinterpret_cast<const char *>(src + begin);
    char *posb = reinterpret_cast<char *>(pos_out + begin);
    const uint32_t len = (uint32_t)(end - begin);
    const uint32_t lastu = len - 1;
    const int32_t Ni = (int32_t)N;  // N < 2^31 (the API's bound)
    auto ld_id = [&](uint32_t o) -> int32_t {
        const uint32_t oc = o < lastu ? o : lastu;
        const int32_t t = __builtin_nontemporal_load(reinterpret_cast<const int32_t *>(srcb + (oc << 2)));
        return o < len ? t : -1;
    };
    // columns per group: the direct form (no staging, fewer registers) keeps
    // 16 columns of IDs in flight (stress batch 9 % faster than with 8; 32
    // were slower), the staged form 8 (16 measured the same)
    constexpr int U = STAGED ? 8 : 16;
    // the IDs of the next U columns load while the current ones are ranked
    // (the loads are unconditional, from a clamped index, so that the wait
    // for a group's IDs does not also wait for the next group's)
    int32_t nxt[U];
#pragma unroll
    for (int u = 0; u < U; u++) nxt[u] = ld_id((uint32_t)(u * kWave + lane));
    // whole groups of U columns store every pair's position unconditionally:
    // a store under a branch leaves the compiler unable to count the stores
    // issued after the prefetched ID loads, and its wait for those loads then
    // also waits for every store (stores and loads share one counter here)
    auto group = [&](int64_t g, auto fullc) {
        constexpr bool FULL = decltype(fullc)::value;
        int32_t v[U];
        const uint32_t go = (uint32_t)(g - begin);
#pragma unroll
        for (int u = 0; u < U; u++) v[u] = nxt[u];
        if (go + 2 * U * kWave <= len) {
            // the next group is whole: one address, the columns at immediate offsets
            const int32_t *q = reinterpret_cast<const int32_t *>(srcb + ((go + U * kWave + (uint32_t)lane) << 2));
#pragma unroll
            for (int u = 0; u < U; u++) nxt[u] = __builtin_nontemporal_load(q + u * kWave);
        } else {
#pragma unroll
            for (int u = 0; u < U; u++) nxt[u] = ld_id(go + (uint32_t)((U + u) * kWave + lane));
        }
        int32_t *pq = reinterpret_cast<int32_t *>(posb + ((go + (uint32_t)lane) << 2));
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
                atomicOr(reinterpret_cast<unsigned long long *>(&mk0[ia]), bit);
                atomicOr(reinterpret_cast<unsigned long long *>(&mk1[ib]), bit);
                wave_lds_fence();
                Cell2 ca, cb;
                ca.mask = mk0[ia];
                ca.mask1 = mk1[ia];
                {
                    const uint2 t = inf[ia];
                    ca.kf = t.x;
                    ca.base = (int32_t)t.y;
                }
                cb.mask = mk0[ib];
                cb.mask1 = mk1[ib];
                {
                    const uint2 t = inf[ib];
                    cb.kf = t.x;
                    cb.base = (int32_t)t.y;
                }
                wave_lds_fence();
                const uint64_t belowa = ca.mask & lt;
                const uint64_t belowb = cb.mask1 & lt;
                // one lane per expert of the pair: its lowest in the first column,
                // else (absent there) its lowest in the second
                if (belowa == 0) {
                    const uint32_t n = (uint32_t)__popcll(ca.mask) + (uint32_t)__popcll(ca.mask1);
                    mk0[ia] = 0ull;
                    mk1[ia] = 0ull;
                    inf[ia] = make_uint2(ca.kf + n, (uint32_t)ca.base + n);
                }
                if (cb.mask == 0 && belowb == 0) {
                    const uint32_t n = (uint32_t)__popcll(cb.mask1);
                    mk1[ib] = 0ull;
                    inf[ib] = make_uint2(cb.kf + n, (uint32_t)cb.base + n);
                }
                const int32_t ka = (int32_t)__popcll(belowa);
                const int32_t kb = (int32_t)__popcll(cb.mask) + (int32_t)__popcll(belowb);
                auto place = [&](const Cell2 &c, int xi, bool valid, int32_t k, int col) {
                    const uint32_t o = go + (uint32_t)(col * kWave + lane);
                    int32_t pos = (c.kf & (kNoneFlag | kSplitFlag)) ? -1 : c.base + k;
                    if (c.kf & kSplitFlag) pos = position_of(inst, rfirst[xi], rcnt[xi], c.base + k);
                    if (STAGED) stage[valid ? (int32_t)(c.kf & kCountMask) + k : sub] = (uint16_t)o;
                    else if ((uint32_t)pos < (uint32_t)Ni) src_out[pos] = (int32_t)(begin + o);
                    if (FULL) __builtin_nontemporal_store(pos, pq + col * kWave);
                    else if (o < len) __builtin_nontemporal_store(pos, reinterpret_cast<int32_t *>(posb + (o << 2)));
                };
                place(ca, ia, va, ka, u);
                place(cb, ib, vb, kb, u + 1);
                wave_lds_fence();
            }
    
        } else {
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int32_t x = v[u];
                const bool valid = (uint32_t)x < uE;
                const int xi = valid ? x : E;  // padding and bad IDs rank in the sink cell
                atomicOr(reinterpret_cast<unsigned long long *>(&mk0[xi]), bit);
                wave_lds_fence();
                Cell1 cur;
                cur.mask = mk0[xi];
                {
                    const uint2 t = inf[xi];
                    cur.kf = t.x;
                    cur.base = (int32_t)t.y;
                }
                wave_lds_fence();
                const uint32_t o = go + (uint32_t)(u * kWave + lane);
                const uint64_t below = cur.mask & lt;
                if (below == 0) {
                    const uint32_t n = (uint32_t)__popcll(cur.mask);
                    mk0[xi] = 0ull;
                    inf[xi] = make_uint2(cur.kf + n, (uint32_t)cur.base + n);
                }
                const int32_t k = (int32_t)__popcll(below);
                int32_t pos = (cur.kf & (kNoneFlag | kSplitFlag)) ? -1 : cur.base + k;
                if (cur.kf & kSplitFlag) pos = position_of(inst, rfirst[xi], rcnt[xi], cur.base + k);
                if (STAGED) stage[valid ? (int32_t)(cur.kf & kCountMask) + k : sub] = (uint16_t)o;
                else if ((uint32_t)pos < (uint32_t)Ni) src_out[pos] = (int32_t)(begin + o);
                if (FULL) __builtin_nontemporal_store(pos, pq + u * kWave);
                else if (o < len) __builtin_nontemporal_store(pos, reinterpret_cast<int32_t *>(posb + (o << 2)));
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
        // staged slots in order, 64 per step; each expert's slots go to
        // consecutive positions (per instance), so every store writes a few
        // coalesced runs
        constexpr int UF = 4;  // windows per step: their LDS reads overlap
        int cbase = 0;  // cells ended before the current window
        for (int w0 = 0; w0 < staged_pairs; w0 += UF * kWave) {
            uint64_t word[UF];
            int cb[UF];
#pragma unroll
            for (int u = 0; u < UF; u++) {
                const int wi = w0 / kWave + u;  // (32-bit: a scalar compare)
                word[u] = wi < (int)nwords ? sbits[wi] : 0ull;
            }
#pragma unroll
            for (int u = 0; u < UF; u++) {
                cb[u] = cbase;
                cbase += __popcll(word[u]);
            }
            // slot t belongs to the c-th non-empty cell, c = the cells that
            // end before t (those of earlier windows plus the end bits of
            // lower lanes).  Every lane reads (a slot past the staged pairs
            // reads a stale slot and cell ncells, whose entry is a valid
            // expert), and only the store is conditional: reads under a
            // branch each got a wait of their own.
            int2 ci[UF];
            uint32_t sidx[UF];
#pragma unroll
            for (int u = 0; u < UF; u++) {
                const int t = w0 + u * kWave + lane;
                const int c = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(word[u] >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)word[u], (uint32_t)cb[u]));
                ci[u] = cinfo[c];
                sidx[u] = stage[(uint32_t)t < (uint32_t)sub ? t : sub];
            }
#pragma unroll
            for (int u = 0; u < UF; u++) {
                const int t = w0 + u * kWave + lane;
                const uint32_t f = (uint32_t)ci[u].y;
                int32_t pos = (f & kNoneFlag) ? -1 : ci[u].x + t;
                if (f & kSplitFlag) {
                    const int ex = (int)(f & kCountMask);
                    pos = position_of(inst, rfirst[ex], rcnt[ex], pos);
                }
                // (a slot past the staged pairs reads record ncells, "none")
                if ((uint32_t)pos < (uint32_t)Ni) src_out[pos] = (int32_t)(begin + sidx[u]);
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
    const size_t staged = stage_pairs > 0 ? (size_t)waves * ((size_t)stage_pairs / kWave * 8 + (size_t)E * 8 + 8 +
                                                             ((size_t)stage_pairs + kWave) * 2) + 8
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
