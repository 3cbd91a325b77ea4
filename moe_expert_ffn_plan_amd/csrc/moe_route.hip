// Routing tables for one GPU's experts: counts, block-padded offsets, slot
// table, inverse tables, per-block expert/slack and the pull order.
//
// What is built follows the fused-MoE practice page (section 2, "schedule
// tables") and the MegaMoE dispatch counting (walk-through section 4.2):
// hits of each local expert are laid out contiguously, each expert's row
// count rounded up to block_m, with a prefix sum over experts.  Rows of one
// expert follow ascending flat hit order t*k + j, so the tables are
// deterministic (the pages' kernels take slots with atomics instead).
//
// Design: one 1024-thread workgroup (16 waves) for up to 4096 hits.  The
// local expert id of every hit is first staged in LDS as int16; every later
// pass reads it from there.  Each wave owns a contiguous range of hits (and
// of tokens, for the pull order).  Pass 1 counts hits per (wave, expert) and
// tokens per (wave, smallest local expert) with LDS atomics; pass 2 turns
// those into per-wave bases with a scan over waves and block-wide scans over
// experts; pass 3 re-walks each wave's hits in order, 64 at a time, and
// ranks equal experts inside the batch with a ballot "match" over the bits
// of the expert id, so every hit's row is its expert's base plus the number
// of earlier hits of that expert.  The pull order is the same counting sort
// of tokens keyed by their smallest local expert (a token's smallest slot
// lies in the range of its smallest expert, and tokens of one expert are in
// ascending t there).  The scans use DPP lane moves, not LDS shuffles.
//
// Larger inputs spread over many CUs in groups of route_group_tokens(T)
// tokens (64, or up to 256 so that there are at most 256 groups where
// possible; one token per lane of a group's four waves): route_count_kernel (per group: hit counts per expert and pull
// counts per smallest expert), then route_scatter_scan_kernel (per group:
// the bases of its group from the counts of all groups, the counts, padded
// offsets, block tables and tile lists, and the same stable ballot-match
// scatter).  Beyond kFusedScanMaxWords group x expert counters the scan runs
// as one workgroup of its own (route_scan_kernel) between the counting and
// the scatter (route_scatter_kernel).  All paths produce identical tables.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// Workgroup barrier for LDS traffic only.  Apart from route_scan_kernel, these kernels never read global
// memory that another thread of the same launch wrote, so their barriers need not wait for outstanding
// global stores the way __syncthreads does (a round trip to memory per barrier, after every pass that
// writes tables).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The single launch's prepare work, when the plan asks for it (PlanPtrs' epoch_word and status): one
// thread advances the launch counter and clears the status word, as the fused prepare kernel does.
__device__ __forceinline__ void plan_prepare(const PlanPtrs& p) {
    if (p.epoch_word && blockIdx.x == 0 && threadIdx.x == 0) {
        const uint32_t v = __hip_atomic_load(p.epoch_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.epoch_word, v + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.status, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Wave-level inclusive scans with DPP lane moves (a few cycles each; a __shfl_up goes through the LDS
// crossbar at LDS latency).  Lanes whose source lies outside the row read 0.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp_add(int v) {
    return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
// within each row of 16 lanes
__device__ __forceinline__ int row_inclusive_scan(int v) {
    v = dpp_add<0x111>(v);  // row_shr:1
    v = dpp_add<0x112>(v);  // row_shr:2
    v = dpp_add<0x114>(v);  // row_shr:4
    return dpp_add<0x118>(v);  // row_shr:8
}
// across the 64 lanes: the row scans, then lane 15 of each row into the next row and lane 31 into the
// upper half
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    v = row_inclusive_scan(v);
    v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    return dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
}

__device__ __forceinline__ uint64_t lanes_lt() { return (1ull << (threadIdx.x & 63)) - 1ull; }

// Lanes of this wave whose `valid` key equals mine (only meaningful if valid).
__device__ __forceinline__ uint64_t match_peers(bool valid, int key, int nbits) {
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t ones = __ballot(valid && bit);
        peers &= bit ? ones : ~ones;
    }
    return peers;
}

// Inclusive scan of one value per thread across the workgroup.
__device__ int block_inclusive_scan(int v, int* scratch) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
    v = wave_inclusive_scan(v);
    if (lane == 63) scratch[wave] = v;
    lds_barrier();
    if (wave == 0) {
        const int t = wave_inclusive_scan(lane < waves ? scratch[lane] : 0);
        if (lane < waves) scratch[lane] = t;
    }
    lds_barrier();
    if (wave > 0) v += scratch[wave - 1];
    lds_barrier();
    return v;
}

// Inclusive scans of N values per thread across the workgroup, sharing one set of barriers.
// scratch: N * 64 ints.
template <int N>
__device__ void block_inclusive_scan_n(int (&v)[N], int* scratch) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = wave_inclusive_scan(v[i]);
    if (lane == 63)
#pragma unroll
        for (int i = 0; i < N; ++i) scratch[i * 64 + wave] = v[i];
    lds_barrier();
    if (wave == 0)
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int t = wave_inclusive_scan(lane < waves ? scratch[i * 64 + lane] : 0);
            if (lane < waves) scratch[i * 64 + lane] = t;
        }
    lds_barrier();
    if (wave > 0)
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] += scratch[i * 64 + wave - 1];
    lds_barrier();
}

// Per-wave counters cnt[w * E + e] (w < W) turned in place into each wave's exclusive prefix over
// the waves before it, with totals[e] = the sum over all W waves.  Thread t handles wave t % W of
// expert t / W (W = 16 lanes per expert: one DPP row scan).  No barrier inside: callers synchronise
// before and after.
template <int W>
__device__ void wave_prefix(int32_t* cnt, int E, int32_t* totals) {
    static_assert(W == 16, "one DPP row of 16 lanes per expert");
    const int ww = threadIdx.x & (W - 1);
    const int per = blockDim.x / W;  // experts per pass
    for (int e0 = 0; e0 < E; e0 += per) {  // the same trip count for every thread (convergent shuffles)
        const int e = e0 + (int)threadIdx.x / W;
        const int c = e < E ? cnt[ww * E + e] : 0;
        const int v = row_inclusive_scan(c);
        if (e < E) {
            cnt[ww * E + e] = v - c;
            if (ww == W - 1) totals[e] = v;
        }
    }
}


// GEMM tile lists from the padded offsets soff (LDS, E+1) and the hit counts scnt (LDS, E).  An M-tile
// covers up to bmg rows of one expert, cut from the expert's first row; expert e has ceil(count / bmg)
// M-tiles, so a tile that would hold only padding rows is not listed (with blocks of 96 or 192 rows an
// expert's padding can exceed a 128-row tile), and a tile's row count stops at the expert's last hit.
// The M-tile counts' exclusive prefix over experts goes to tb (LDS scratch, E+1), so M-tiles are
// numbered expert by expert.  For a GEMM with nt N-tiles the list runs M-tile by M-tile, all N-tiles
// of each: entry l = mt * nt + n = {first row, n << 16 | e, valid rows, mt}.  A range of M-tiles is
// then a contiguous range of both GEMMs' lists.  Called by every thread of the workgroup; workgroup
// `part` of `parts` writes the entries l with l / blockDim.x = part mod parts.  scalars[4], [5] =
// tiles of each GEMM (if `counts`).
__device__ void write_tile_lists(const int32_t* soff, const int32_t* scnt, int E, int32_t* tb, const PlanPtrs& p,
                                 int part, int parts, bool counts) {
    const int bmg = p.bmg;
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int run = 0;
        for (int c = 0; c < E; c += 64) {
            const int e = c + lane;
            int v = 0;
            if (e < E) v = (scnt[e] + bmg - 1) / bmg;
            v = wave_inclusive_scan(v);
            if (e < E) tb[e + 1] = run + v;
            run += __builtin_amdgcn_readlane(v, 63);
        }
        if (lane == 0) tb[0] = 0;
    }
    lds_barrier();
    const int mt_total = tb[E];
    if (counts && threadIdx.x == 0) {
        p.scalars[4] = mt_total * p.nt1;
        p.scalars[5] = mt_total * p.nt2;
    }
    for (int pass = 0; pass < 2; ++pass) {
        const int nt = pass == 0 ? p.nt1 : p.nt2;
        int32_t* tiles = pass == 0 ? p.tiles1 : p.tiles2;
        const int total = mt_total * nt;
        for (int l = part * blockDim.x + threadIdx.x; l < total; l += parts * blockDim.x) {
            const int mt = l / nt, n = l - mt * nt;
            int lo = 0, hi = E - 1;  // the expert of M-tile mt: largest e with tb[e] <= mt
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (tb[mid] <= mt) lo = mid; else hi = mid - 1;
            }
            const int m0 = soff[lo] + (mt - tb[lo]) * bmg;
            int32_t* t = tiles + (size_t)kTileWords * l;
            t[0] = m0;
            t[1] = (n << 16) | lo;
            t[2] = min(bmg, soff[lo] + scnt[lo] - m0);
            t[3] = mt;
        }
    }
}

// Largest input the one-workgroup kernel can hold (its local expert ids sit in LDS as int16), and the
// size up to which it is used: beyond a few thousand hits its scattered table stores from a single CU
// cost more than the extra launch of the multi-workgroup path.
constexpr int kSingleMaxHits = 32768;
constexpr int kSingleWorkgroupHits = 4096;

__global__ __launch_bounds__(kThreads) void route_kernel(const int64_t* __restrict__ ids, int T, int k, int E,
                                                         int expert_begin, int bm, PlanPtrs p) {
    __shared__ int16_t le[kSingleMaxHits];        // local expert of every hit, -1 if not local
    __shared__ int32_t wcnt[kWaves * kMaxExperts]; // per-wave hit counters, later per-wave bases
    __shared__ int32_t wpc[kWaves * kMaxExperts];  // per-wave pull counters, later per-wave bases
    __shared__ int32_t soff[kMaxExperts + 1];      // padded offsets
    __shared__ int32_t scnt[kMaxExperts];          // counts
    __shared__ int32_t sbase[kMaxExperts + 1];     // pull totals, then pull-order bases
    __shared__ int32_t tb[kMaxExperts + 1];        // M-tile bases per expert
    __shared__ int32_t scratch[192];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    const int64_t begin = expert_begin;
    const int nh = T * k;
    plan_prepare(p);

    // ---- pass 0: ids -> local experts in LDS (8 loads in flight per thread), counters cleared
    for (int base = 0; base < nh; base += 8 * kThreads) {
        int64_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int h = base + u * kThreads + tid;
            v[u] = h < nh ? ids[h] - begin : -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int h = base + u * kThreads + tid;
            if (h < nh) le[h] = (int16_t)((v[u] >= 0 && v[u] < E) ? v[u] : -1);
        }
    }
    for (int i = tid; i < kWaves * E; i += kThreads) {
        wcnt[i] = 0;
        wpc[i] = 0;
    }
    lds_barrier();

    // ---- pass 1: hits per (wave, expert), wave w owning the contiguous hits [h0, h1); and tokens per
    // (wave, smallest local expert), wave w owning the contiguous tokens [t0, t1) (for the pull order)
    const int per_wave = (nh + kWaves * 64 - 1) / (kWaves * 64) * 64;
    const int h0 = min(nh, w * per_wave);
    const int h1 = min(nh, h0 + per_wave);
    for (int h = h0 + lane; h < h1; h += 64) {
        const int e = le[h];
        if (e >= 0) atomicAdd(&wcnt[w * E + e], 1);
    }
    const int tper = (T + kWaves * 64 - 1) / (kWaves * 64) * 64;
    const int t0 = min(T, w * tper), t1 = min(T, t0 + tper);
    auto smallest = [&](int t) {
        int emin = E;
        for (int j = 0; j < k; ++j) {
            const int e = le[t * k + j];
            if (e >= 0 && e < emin) emin = e;
        }
        return emin;
    };
    for (int base = t0; base < t1; base += 64) {
        const int t = base + lane;
        const int emin = t < t1 ? smallest(t) : E;
        if (emin < E) atomicAdd(&wpc[w * E + emin], 1);
    }
    lds_barrier();

    // ---- pass 2: per-wave bases, counts, padded offsets, pull bases
    wave_prefix<kWaves>(wcnt, E, scnt);
    wave_prefix<kWaves>(wpc, E, sbase + 1);  // pull totals for now
    lds_barrier();
    const int cnt = tid < E ? scnt[tid] : 0;
    int sv[3] = {(cnt + bm - 1) / bm * bm, cnt, tid < E ? sbase[tid + 1] : 0};
    block_inclusive_scan_n<3>(sv, scratch);
    const int incl_pad = sv[0], incl_cnt = sv[1], incl_pull = sv[2];
    if (tid < E) {
        soff[tid + 1] = incl_pad;
        sbase[tid + 1] = incl_pull;
        p.counts[tid] = cnt;
        p.offsets[tid + 1] = incl_pad;
    }
    if (tid == 0) {
        soff[0] = 0;
        sbase[0] = 0;
        p.offsets[0] = 0;
    }
    if (tid == E - 1) {
        p.scalars[0] = incl_pad;        // R_pad
        p.scalars[1] = incl_pull;       // n_pull
        p.scalars[2] = incl_cnt;        // N
        p.scalars[3] = incl_pad / bm;   // n_blocks
    }
    lds_barrier();

    // ---- pass 3: stable scatter of hits into rows, 64 at a time in flat order
    for (int base = h0; base < h1; base += 64) {
        const int h = base + lane;
        const int e = h < h1 ? le[h] : -1;
        const bool valid = e >= 0;
        const uint64_t peers = match_peers(valid, e, nbits);
        if (valid) {
            const int rank = __popcll(peers & lanes_lt());
            const int cur = wcnt[w * E + e];
            const int row = soff[e] + cur + rank;
            p.slot[h] = row;
            p.row_token[row] = h / k;
            p.row_topk[row] = h % k;
            if (rank == 0) wcnt[w * E + e] = cur + __popcll(peers);
        } else if (h < h1) {
            p.slot[h] = -1;
        }
    }

    // ---- pass 4: per-block expert and slack; padding rows marked -1; GEMM tile lists
    const int r_pad = soff[E];
    const int n_blocks = r_pad / bm;
    for (int b = tid; b < n_blocks; b += kThreads) {
        const int r = b * bm;
        int lo = 0, hi = E;  // largest e with soff[e] <= r (that expert has rows, so soff[e+1] > r)
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (soff[mid] <= r) lo = mid; else hi = mid - 1;
        }
        const int e = lo;
        const int fill_end = soff[e] + scnt[e];
        const int valid_rows = max(0, min(r + bm, fill_end) - max(r, soff[e]));
        p.block_expert[b] = e;
        p.slack[b] = bm - valid_rows;
        for (int q = max(r, fill_end); q < r + bm; ++q) {
            p.row_token[q] = -1;
            p.row_topk[q] = -1;
        }
    }
    write_tile_lists(soff, scnt, E, tb, p, 0, 1, true);
    lds_barrier();

    // ---- pass 5: pull order = tokens with a hit, by smallest local expert, then t (bases from pass 2)
    for (int base = t0; base < t1; base += 64) {
        const int t = base + lane;
        const int emin = t < t1 ? smallest(t) : E;
        const bool valid = emin < E;
        const uint64_t peers = match_peers(valid, emin, nbits);
        if (valid) {
            const int rank = __popcll(peers & lanes_lt());
            const int cur = wpc[w * E + emin];
            p.pull_order[sbase[emin] + cur + rank] = t;
            if (rank == 0) wpc[w * E + emin] = cur + __popcll(peers);
        }
    }
}

// ---------------------------------------------------------------- multi-group path
constexpr int kGThreads = 256;
constexpr int kGWaves = kGThreads / 64;

// Loads the group's top-k ids once (coalesced, 8 loads in flight per thread) as local expert
// ids, -1 when not local, into LDS `le` [tokens * k].
__device__ __forceinline__ void load_group_experts(const int64_t* __restrict__ ids, int64_t h0, int64_t h1, int k,
                                                   int64_t begin, int E, int16_t* le) {
    const int n = (int)(h1 - h0);
    for (int base = 0; base < n; base += 8 * kGThreads) {
        int64_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = base + u * kGThreads + threadIdx.x;
            v[u] = i < n ? ids[h0 + i] - begin : -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = base + u * kGThreads + threadIdx.x;
            if (i < n) le[i] = (int16_t)((v[u] >= 0 && v[u] < E) ? v[u] : -1);
        }
    }
}

// The same in two steps, so that other global loads can be in flight together with these: fetch_ids
// issues the loads of the first 8 * kGThreads hits into registers, store_ids converts and writes them
// (and handles any further hits as load_group_experts does).
__device__ __forceinline__ void fetch_ids(const int64_t* __restrict__ ids, int64_t h0, int n, int64_t (&v)[8]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int i = u * kGThreads + threadIdx.x;
        v[u] = i < n ? ids[h0 + i] : -1;
    }
}
__device__ __forceinline__ void store_ids(const int64_t* __restrict__ ids, int64_t h0, int n, const int64_t (&v)[8],
                                          int64_t begin, int E, int16_t* le) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int i = u * kGThreads + threadIdx.x;
        const int64_t e = v[u] - begin;
        if (i < n) le[i] = (int16_t)((e >= 0 && e < E) ? e : -1);
    }
    if (n > 8 * kGThreads) load_group_experts(ids, h0 + 8 * kGThreads, h0 + n, 0, begin, E, le + 8 * kGThreads);
}

__device__ __forceinline__ int smallest_in(const int16_t* le, int t_local, int k, int E) {
    int emin = E;
    for (int j = 0; j < k; ++j) {
        const int e = le[t_local * k + j];
        if (e >= 0 && e < emin) emin = e;
    }
    return emin;
}

// group_counts: [groups][E] hit counts, then [groups][E] pull counts.
__global__ __launch_bounds__(kGThreads) void route_count_kernel(const int64_t* __restrict__ ids, int T, int k, int E,
                                                               int expert_begin, int groups, int tpg,
                                                               int32_t* __restrict__ gcounts) {
    extern __shared__ int32_t lds[];
    int32_t* ch = lds;                                          // [E]
    int32_t* cp = lds + E;                                      // [E]
    int16_t* le = reinterpret_cast<int16_t*>(lds + 2 * E);      // [tpg * k]
    const int tid = threadIdx.x, g = blockIdx.x;
    for (int i = tid; i < 2 * E; i += kGThreads) lds[i] = 0;
    const int t0 = g * tpg, t1 = min(T, t0 + tpg);
    load_group_experts(ids, (int64_t)t0 * k, (int64_t)t1 * k, k, expert_begin, E, le);
    lds_barrier();
    const int nh = (t1 - t0) * k;
    for (int i = tid; i < nh; i += kGThreads)
        if (le[i] >= 0) atomicAdd(&ch[le[i]], 1);
    for (int t = tid; t < t1 - t0; t += kGThreads) {
        const int emin = smallest_in(le, t, k, E);
        if (emin < E) atomicAdd(&cp[emin], 1);
    }
    lds_barrier();
    for (int e = tid; e < E; e += kGThreads) {
        gcounts[(size_t)g * E + e] = ch[e];
        gcounts[((size_t)groups + g) * E + e] = cp[e];
    }
}

// One workgroup: turns group counts into absolute group bases (slot row and pull position of the
// group's first hit / token of each expert), and writes counts, offsets, scalars, block tables and
// the padding rows.  Group counts go through LDS in chunks of whole groups.
constexpr int kScanChunkWords = 8192;

__global__ __launch_bounds__(kThreads) void route_scan_kernel(int E, int bm, int groups, int32_t* __restrict__ gcounts,
                                                             PlanPtrs p) {
    plan_prepare(p);
    extern __shared__ int32_t lds[];
    int32_t* soff = lds;            // [E+1] padded offsets
    int32_t* scnt = soff + E + 1;   // [E] hit counts
    int32_t* pbase = scnt + E;      // [E+1] pull bases
    int32_t* ptot = pbase + E + 1;  // [E] pull counts
    int32_t* scratch = ptot + E;    // [64]
    int32_t* tb = scratch + 64;     // [E+1] M-tile bases
    int32_t* chunk = tb + E + 1;    // [kScanChunkWords]
    const int tid = threadIdx.x;
    const int gpc = max(1, kScanChunkWords / (2 * E));  // groups per chunk
    const bool one_chunk = groups <= gpc;               // then the group prefixes stay in LDS
    int run = 0, prun = 0;                              // running sums of expert `tid`
    for (int g0 = 0; g0 < groups; g0 += gpc) {
        const int ng = min(gpc, groups - g0);
        for (int i = tid; i < ng * E; i += kThreads) {
            chunk[i] = gcounts[(size_t)g0 * E + i];
            chunk[ng * E + i] = gcounts[((size_t)groups + g0) * E + i];
        }
        __syncthreads();
        if (tid < E)
            for (int g = 0; g < ng; ++g) {
                const int c = chunk[g * E + tid], cq = chunk[(ng + g) * E + tid];
                chunk[g * E + tid] = run;
                chunk[(ng + g) * E + tid] = prun;
                run += c;
                prun += cq;
            }
        __syncthreads();
        if (!one_chunk) {
            for (int i = tid; i < ng * E; i += kThreads) {
                gcounts[(size_t)g0 * E + i] = chunk[i];
                gcounts[((size_t)groups + g0) * E + i] = chunk[ng * E + i];
            }
            __syncthreads();
        }
    }
    if (tid < E) {
        scnt[tid] = run;
        ptot[tid] = prun;
    }
    const int cnt = tid < E ? run : 0;
    const int padded = (cnt + bm - 1) / bm * bm;
    const int incl_pad = block_inclusive_scan(padded, scratch);
    const int incl_cnt = block_inclusive_scan(cnt, scratch);
    const int incl_pull = block_inclusive_scan(tid < E ? prun : 0, scratch);
    if (tid < E) {
        soff[tid + 1] = incl_pad;
        pbase[tid + 1] = incl_pull;
        p.counts[tid] = cnt;
        p.offsets[tid + 1] = incl_pad;
    }
    if (tid == 0) {
        soff[0] = 0;
        pbase[0] = 0;
        p.offsets[0] = 0;
    }
    if (tid == E - 1) {
        p.scalars[0] = incl_pad;        // R_pad
        p.scalars[1] = incl_pull;       // n_pull
        p.scalars[2] = incl_cnt;        // N
        p.scalars[3] = incl_pad / bm;   // n_blocks
    }
    __syncthreads();
    if (one_chunk) {
        for (int i = tid; i < groups * E; i += kThreads) {
            const int e = i % E;
            gcounts[i] = chunk[i] + soff[e];
            gcounts[(size_t)groups * E + i] = chunk[groups * E + i] + pbase[e];
        }
    } else {
        for (int64_t i = tid; i < (int64_t)groups * E; i += kThreads) {
            const int e = (int)(i % E);
            gcounts[i] += soff[e];
            gcounts[(size_t)groups * E + i] += pbase[e];
        }
    }
    const int n_blocks = soff[E] / bm;
    for (int b = tid; b < n_blocks; b += kThreads) {
        const int r = b * bm;
        int lo = 0, hi = E;  // largest e with soff[e] <= r (that expert has rows)
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (soff[mid] <= r) lo = mid; else hi = mid - 1;
        }
        const int fill_end = soff[lo] + scnt[lo];
        p.block_expert[b] = lo;
        p.slack[b] = bm - max(0, min(r + bm, fill_end) - max(r, soff[lo]));
        for (int q = max(r, fill_end); q < r + bm; ++q) {
            p.row_token[q] = -1;
            p.row_topk[q] = -1;
        }
    }
    write_tile_lists(soff, scnt, E, tb, p, 0, 1, true);
}

__global__ __launch_bounds__(kGThreads) void route_scatter_kernel(const int64_t* __restrict__ ids, int T, int k, int E,
                                                                 int expert_begin, int groups, int tpg,
                                                                 const int32_t* __restrict__ gcounts, PlanPtrs p) {
    extern __shared__ int32_t lds[];
    int32_t* wh = lds;                                           // [kGWaves][E] running hit rows
    int32_t* wp = lds + kGWaves * E;                             // [kGWaves][E] running pull positions
    int16_t* le = reinterpret_cast<int16_t*>(lds + 2 * kGWaves * E);  // [tpg * k]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = blockIdx.x;
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    for (int i = tid; i < 2 * kGWaves * E; i += kGThreads) lds[i] = 0;
    const int tg0 = g * tpg, tg1 = min(T, tg0 + tpg);
    load_group_experts(ids, (int64_t)tg0 * k, (int64_t)tg1 * k, k, expert_begin, E, le);
    __syncthreads();
    const int wt = tpg / kGWaves;                  // tokens per wave, at most 64
    const int t0 = min(tg1, tg0 + w * wt);  // this wave's tokens [t0, t1)
    const int t1 = min(tg1, t0 + wt);
    const int l0 = (t0 - tg0) * k, l1 = (t1 - tg0) * k;  // and hits (group-local)
    for (int i = l0 + lane; i < l1; i += 64)
        if (le[i] >= 0) atomicAdd(&wh[w * E + le[i]], 1);
    const int tt = t0 + lane;
    const int emin = tt < t1 ? smallest_in(le, tt - tg0, k, E) : E;
    if (emin < E) atomicAdd(&wp[w * E + emin], 1);
    __syncthreads();
    for (int e = tid; e < E; e += kGThreads) {
        int run = gcounts[(size_t)g * E + e];
        int prun = gcounts[((size_t)groups + g) * E + e];
        for (int ww = 0; ww < kGWaves; ++ww) {
            const int c = wh[ww * E + e], cq = wp[ww * E + e];
            wh[ww * E + e] = run;
            wp[ww * E + e] = prun;
            run += c;
            prun += cq;
        }
    }
    __syncthreads();
    // stable scatter of this wave's hits (flat order), 64 at a time
    const int64_t hg0 = (int64_t)tg0 * k;
    for (int base = l0; base < l1; base += 64) {
        const int i = base + lane;
        const int e = i < l1 ? le[i] : -1;
        const bool valid = e >= 0;
        const uint64_t peers = match_peers(valid, e, nbits);
        const int64_t h = hg0 + i;
        if (valid) {
            const int rank = __popcll(peers & lanes_lt());
            const int cur = wh[w * E + e];
            const int row = cur + rank;
            p.slot[h] = row;
            p.row_token[row] = (int)(h / k);
            p.row_topk[row] = (int)(h % k);
            if (rank == 0) wh[w * E + e] = cur + __popcll(peers);
        } else if (i < l1) {
            p.slot[h] = -1;
        }
    }
    // pull order: this wave's tokens by smallest local expert, ascending t
    const bool pv = emin < E;
    const uint64_t peers = match_peers(pv, emin, nbits);
    if (pv) {
        const int rank = __popcll(peers & lanes_lt());
        p.pull_order[wp[w * E + emin] + rank] = tt;
    }
}

// Count-then-scatter path without a separate scan: every scatter workgroup reads the whole table of
// per-group counts (groups x E hit counts and pull counts, small for the inputs it is used for) and
// computes the scan itself, so all of them agree on the offsets; workgroup g then scatters its own
// group, and the workgroups share the block tables, padding rows and tile lists by striding.
constexpr int kFusedScanMaxWords = 65536;  // groups * E up to this takes the two-kernel path

__global__ __launch_bounds__(kGThreads) void route_scatter_scan_kernel(const int64_t* __restrict__ ids, int T, int k,
                                                                      int E, int expert_begin, int groups, int tpg,
                                                                      int bm, const int32_t* __restrict__ gcounts,
                                                                      PlanPtrs p) {
    plan_prepare(p);
    extern __shared__ int32_t lds[];
    int32_t* wh = lds;                      // [kGWaves][E] running hit rows
    int32_t* wp = wh + kGWaves * E;         // [kGWaves][E] running pull positions
    int32_t* soff = wp + kGWaves * E;       // [E+1] padded offsets
    int32_t* scnt = soff + E + 1;           // [E] hit counts (all groups)
    int32_t* pbase = scnt + E;              // [E+1] pull bases
    int32_t* gh = pbase + E + 1;            // [E] this group's first row of each expert (before soff)
    int32_t* gp = gh + E;                   // [E] this group's first pull position (before pbase)
    int32_t* scratch = gp + E;              // [192]
    int32_t* tb = scratch + 192;            // [E+1] M-tile bases
    int32_t* part = tb + E + 1;             // [4][kGThreads] partial sums of the group-count scan
    int16_t* le = reinterpret_cast<int16_t*>(part + 4 * kGThreads);  // [tpg * k]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = blockIdx.x;
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    for (int i = tid; i < 2 * kGWaves * E; i += kGThreads) lds[i] = 0;
    const int tg0 = g * tpg, tg1 = min(T, tg0 + tpg);
    const int nh = (tg1 - tg0) * k;
    int64_t idv[8];
    fetch_ids(ids, (int64_t)tg0 * k, nh, idv);  // in flight during the group-count loads below

    // ---- scan of the group counts: totals and this group's bases per expert.  With E <= 256 the
    // threads split as (expert, slice of the groups), each summing every nsl-th group with several
    // loads in flight, and the slices are combined through LDS; larger E loop over the experts.
    {
        const int nsl = E <= kGThreads ? kGThreads / E : 1;
        for (int e0 = 0; e0 < E; e0 += kGThreads) {
            const int e = e0 + (E <= kGThreads ? tid % E : tid), sl = E <= kGThreads ? tid / E : 0;
            int tot = 0, ptot_ = 0, lt = 0, plt = 0;
            if (e < E && sl < nsl) {
                constexpr int kU = 8;  // loads in flight per thread
                for (int gb = sl; gb < groups; gb += kU * nsl) {
                    int hc[kU], pc[kU];
#pragma unroll
                    for (int u = 0; u < kU; ++u) {
                        const int gg = gb + u * nsl;
                        hc[u] = gg < groups ? gcounts[(size_t)gg * E + e] : 0;
                        pc[u] = gg < groups ? gcounts[((size_t)groups + gg) * E + e] : 0;
                    }
#pragma unroll
                    for (int u = 0; u < kU; ++u) {
                        const int gg = gb + u * nsl;
                        tot += hc[u];
                        ptot_ += pc[u];
                        if (gg < g) { lt += hc[u]; plt += pc[u]; }
                    }
                }
            }
            part[tid] = tot;
            part[kGThreads + tid] = ptot_;
            part[2 * kGThreads + tid] = lt;
            part[3 * kGThreads + tid] = plt;
            lds_barrier();
            if (tid < min(E - e0, kGThreads)) {
                int a = 0, b = 0, c = 0, d = 0;
                for (int q = 0; q < nsl; ++q) {  // slice q of expert e0 + tid sits at thread q * E + tid
                    const int src = E <= kGThreads ? q * E + tid : tid;
                    a += part[src];
                    b += part[kGThreads + src];
                    c += part[2 * kGThreads + src];
                    d += part[3 * kGThreads + src];
                }
                const int e = e0 + tid;
                scnt[e] = a;
                pbase[e + 1] = b;  // pull totals for now
                gh[e] = c;
                gp[e] = d;
            }
            lds_barrier();
        }
    }
    // exclusive scans over experts (E <= 512 = 2 * kGThreads): thread t owns experts 2t and 2t+1
    {
        int padded, pulls, cnt;
        const int e0 = 2 * tid, e1 = 2 * tid + 1;
        const int c0 = e0 < E ? scnt[e0] : 0, c1 = e1 < E ? scnt[e1] : 0;
        const int p0 = e0 < E ? pbase[e0 + 1] : 0, p1 = e1 < E ? pbase[e1 + 1] : 0;
        const int pad0 = (c0 + bm - 1) / bm * bm, pad1 = (c1 + bm - 1) / bm * bm;
        padded = pad0 + pad1;
        pulls = p0 + p1;
        cnt = c0 + c1;
        int sv[3] = {padded, pulls, cnt};
        block_inclusive_scan_n<3>(sv, scratch);
        const int incl_pad = sv[0], incl_pull = sv[1], incl_cnt = sv[2];
        if (e0 < E) { soff[e0 + 1] = incl_pad - pad1; pbase[e0 + 1] = incl_pull - p1; }
        if (e1 < E) { soff[e1 + 1] = incl_pad; pbase[e1 + 1] = incl_pull; }
        if (tid == 0) { soff[0] = 0; pbase[0] = 0; }
        if (g == 0) {
            if (e0 < E) p.counts[e0] = c0;
            if (e1 < E) p.counts[e1] = c1;
            if (tid == (E - 1) / 2) {
                p.scalars[0] = incl_pad;        // R_pad
                p.scalars[1] = incl_pull;       // n_pull
                p.scalars[2] = incl_cnt;        // N
                p.scalars[3] = incl_pad / bm;   // n_blocks
            }
        }
    }
    lds_barrier();
    if (g == 0)
        for (int e = tid; e <= E; e += kGThreads) p.offsets[e] = soff[e];

    store_ids(ids, (int64_t)tg0 * k, nh, idv, expert_begin, E, le);
    lds_barrier();

    // ---- this group's per-wave bases, then the stable scatter (as in route_scatter_kernel)
    const int wt = tpg / kGWaves;  // tokens per wave, at most 64
    const int t0 = min(tg1, tg0 + w * wt);
    const int t1 = min(tg1, t0 + wt);
    const int l0 = (t0 - tg0) * k, l1 = (t1 - tg0) * k;
    for (int i = l0 + lane; i < l1; i += 64)
        if (le[i] >= 0) atomicAdd(&wh[w * E + le[i]], 1);
    const int tt = t0 + lane;
    const int emin = tt < t1 ? smallest_in(le, tt - tg0, k, E) : E;
    if (emin < E) atomicAdd(&wp[w * E + emin], 1);
    lds_barrier();
    for (int e = tid; e < E; e += kGThreads) {
        int run = soff[e] + gh[e], prun = pbase[e] + gp[e];
        for (int ww = 0; ww < kGWaves; ++ww) {
            const int c = wh[ww * E + e], cq = wp[ww * E + e];
            wh[ww * E + e] = run;
            wp[ww * E + e] = prun;
            run += c;
            prun += cq;
        }
    }
    lds_barrier();
    const int64_t hg0 = (int64_t)tg0 * k;
    for (int base = l0; base < l1; base += 64) {
        const int i = base + lane;
        const int e = i < l1 ? le[i] : -1;
        const bool valid = e >= 0;
        const uint64_t peers = match_peers(valid, e, nbits);
        const int64_t h = hg0 + i;
        if (valid) {
            const int rank = __popcll(peers & lanes_lt());
            const int cur = wh[w * E + e];
            const int row = cur + rank;
            p.slot[h] = row;
            p.row_token[row] = (int)(h / k);
            p.row_topk[row] = (int)(h % k);
            if (rank == 0) wh[w * E + e] = cur + __popcll(peers);
        } else if (i < l1) {
            p.slot[h] = -1;
        }
    }
    {
        const bool pv = emin < E;
        const uint64_t peers = match_peers(pv, emin, nbits);
        if (pv) {
            const int rank = __popcll(peers & lanes_lt());
            p.pull_order[wp[w * E + emin] + rank] = tt;
        }
    }

    // ---- shared across workgroups: block tables and padding rows (one wave per expert), tile lists
    const int nw_all = gridDim.x * kGWaves;
    for (int e = g * kGWaves + w; e < E; e += nw_all) {
        const int fill_end = soff[e] + scnt[e], end = soff[e + 1];
        for (int q = fill_end + lane; q < end; q += 64) {
            p.row_token[q] = -1;
            p.row_topk[q] = -1;
        }
        for (int b = soff[e] / bm + lane; b < end / bm; b += 64) {
            const int r = b * bm;
            p.block_expert[b] = e;
            p.slack[b] = bm - max(0, min(r + bm, fill_end) - r);
        }
    }
    write_tile_lists(soff, scnt, E, tb, p, g, gridDim.x, g == 0);
}

}  // namespace

hipError_t launch_route(const moe_shape& s, const int64_t* topk_idx, const PlanPtrs& p, hipStream_t stream) {
    const int E = s.num_experts;
    const int64_t hits = (int64_t)s.num_tokens * s.topk;
    if (hits <= kSingleWorkgroupHits) {
        hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kThreads), 0, stream, topk_idx, s.num_tokens, s.topk, E,
                           s.expert_begin, s.block_m, p);
        return hipGetLastError();
    }
    const int tpg = route_group_tokens(s.num_tokens);
    const int groups = (s.num_tokens + tpg - 1) / tpg;
    const size_t le_bytes = (size_t)tpg * s.topk * 2;
    hipLaunchKernelGGL(route_count_kernel, dim3(groups), dim3(kGThreads), (size_t)2 * E * 4 + le_bytes, stream,
                       topk_idx, s.num_tokens, s.topk, E, s.expert_begin, groups, tpg, p.group_counts);
    if ((int64_t)groups * E <= kFusedScanMaxWords) {
        const size_t lds = (size_t)(2 * kGWaves * E + 6 * E + 3 + 192 + 4 * kGThreads) * 4 + le_bytes;
        hipLaunchKernelGGL(route_scatter_scan_kernel, dim3(groups), dim3(kGThreads), lds, stream, topk_idx,
                           s.num_tokens, s.topk, E, s.expert_begin, groups, tpg, s.block_m, p.group_counts, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kThreads), (size_t)(5 * E + 3 + 64 + kScanChunkWords) * 4,
                       stream, E, s.block_m, groups, p.group_counts, p);
    hipLaunchKernelGGL(route_scatter_kernel, dim3(groups), dim3(kGThreads), (size_t)2 * kGWaves * E * 4 + le_bytes,
                       stream, topk_idx, s.num_tokens, s.topk, E, s.expert_begin, groups, tpg, p.group_counts, p);
    return hipGetLastError();
}

}  // namespace moe
