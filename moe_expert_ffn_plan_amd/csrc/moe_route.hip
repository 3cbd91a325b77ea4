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
// Design: one 1024-thread workgroup (16 waves).  Each wave owns a contiguous
// range of hits.  Pass 1 counts hits per (wave, expert) with LDS atomics;
// pass 2 turns those into per-wave bases with a scan over waves and a
// block-wide scan over experts; pass 3 re-walks each wave's hits in order,
// 64 at a time, and ranks equal experts inside the batch with a ballot
// "match" over the bits of the expert id, so every hit's row is its expert's
// base plus the number of earlier hits of that expert.  The pull order is a
// second counting sort of tokens keyed by their smallest local expert (a
// token's smallest slot lies in the range of its smallest expert, and tokens
// of one expert are in ascending t there).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 4;  // 64-hit batches a lane keeps in flight

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
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    if (lane == 63) scratch[wave] = v;
    __syncthreads();
    if (wave == 0) {
        int t = lane < kWaves ? scratch[lane] : 0;
        for (int d = 1; d < kWaves; d <<= 1) {
            const int o = __shfl_up(t, d, 64);
            if (lane >= d) t += o;
        }
        if (lane < kWaves) scratch[lane] = t;
    }
    __syncthreads();
    if (wave > 0) v += scratch[wave - 1];
    __syncthreads();
    return v;
}

__device__ __forceinline__ int local_expert(const int64_t* ids, int64_t h, int64_t begin, int E) {
    const int64_t le = ids[h] - begin;
    return (le >= 0 && le < E) ? (int)le : -1;
}

__global__ __launch_bounds__(kThreads) void route_kernel(const int64_t* __restrict__ ids, int T, int k, int E,
                                                         int expert_begin, int bm, PlanPtrs p) {
    extern __shared__ int32_t lds[];
    int32_t* wcnt = lds;                 // [kWaves][E] per-wave counters, later per-wave bases
    int32_t* soff = wcnt + kWaves * E;   // [E+1] padded offsets
    int32_t* scnt = soff + E + 1;        // [E] counts
    int32_t* sbase = scnt + E;           // [E+1] pull-order bases
    int32_t* scratch = sbase + E + 1;    // [64]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    const int64_t begin = expert_begin;

    for (int i = tid; i < kWaves * E; i += kThreads) wcnt[i] = 0;
    __syncthreads();

    // ---- pass 1: hits per (wave, expert)
    const int64_t nh = (int64_t)T * k;
    const int64_t per_wave = (nh + kWaves * 64 - 1) / (kWaves * 64) * 64;
    const int64_t h0 = (int64_t)w * per_wave;
    const int64_t h1 = min(nh, h0 + per_wave);
    for (int64_t base = h0; base < h1; base += 64 * kUnroll) {
        int e[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t h = base + u * 64 + lane;
            e[u] = h < h1 ? local_expert(ids, h, begin, E) : -1;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (e[u] >= 0) atomicAdd(&wcnt[w * E + e[u]], 1);
    }
    __syncthreads();

    // ---- pass 2: per-wave bases, counts, padded offsets
    for (int e = tid; e < E; e += kThreads) {
        int run = 0;
        for (int ww = 0; ww < kWaves; ++ww) {
            const int c = wcnt[ww * E + e];
            wcnt[ww * E + e] = run;
            run += c;
        }
        scnt[e] = run;
    }
    __syncthreads();
    const int cnt = tid < E ? scnt[tid] : 0;
    const int padded = (cnt + bm - 1) / bm * bm;
    const int incl_pad = block_inclusive_scan(padded, scratch);
    const int incl_cnt = block_inclusive_scan(cnt, scratch);
    if (tid < E) {
        soff[tid + 1] = incl_pad;
        p.counts[tid] = cnt;
        p.offsets[tid + 1] = incl_pad;
    }
    if (tid == 0) {
        soff[0] = 0;
        p.offsets[0] = 0;
    }
    if (tid == E - 1) {
        p.scalars[0] = incl_pad;        // R_pad
        p.scalars[2] = incl_cnt;        // N
        p.scalars[3] = incl_pad / bm;   // n_blocks
    }
    __syncthreads();

    // ---- pass 3: stable scatter of hits into rows
    for (int64_t base = h0; base < h1; base += 64 * kUnroll) {
        int e[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t h = base + u * 64 + lane;
            e[u] = h < h1 ? local_expert(ids, h, begin, E) : -1;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t h = base + u * 64 + lane;
            const bool valid = e[u] >= 0;
            const uint64_t peers = match_peers(valid, e[u], nbits);
            if (valid) {
                const int rank = __popcll(peers & lanes_lt());
                const int cur = wcnt[w * E + e[u]];
                const int row = soff[e[u]] + cur + rank;
                p.slot[h] = row;
                p.row_token[row] = (int)(h / k);
                p.row_topk[row] = (int)(h % k);
                if (rank == 0) wcnt[w * E + e[u]] = cur + __popcll(peers);
            } else if (h < h1) {
                p.slot[h] = -1;
            }
        }
    }

    // ---- pass 4: per-block expert and slack; padding rows marked -1
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
    __syncthreads();

    // ---- pass 5: pull order = tokens with a hit, by smallest local expert, then t
    for (int i = tid; i < kWaves * E; i += kThreads) wcnt[i] = 0;
    __syncthreads();
    const int tper = (T + kWaves * 64 - 1) / (kWaves * 64) * 64;
    const int t0 = w * tper, t1 = min(T, t0 + tper);
    for (int base = t0; base < t1; base += 64) {
        const int t = base + lane;
        int emin = E;
        if (t < t1)
            for (int j = 0; j < k; ++j) {
                const int e = local_expert(ids, (int64_t)t * k + j, begin, E);
                if (e >= 0 && e < emin) emin = e;
            }
        if (emin < E) atomicAdd(&wcnt[w * E + emin], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) {
        int run = 0;
        for (int ww = 0; ww < kWaves; ++ww) {
            const int c = wcnt[ww * E + e];
            wcnt[ww * E + e] = run;
            run += c;
        }
        scnt[e] = run;  // counts are no longer needed; reuse for pull counts
    }
    __syncthreads();
    const int pc = tid < E ? scnt[tid] : 0;
    const int incl_pull = block_inclusive_scan(pc, scratch);
    if (tid < E) sbase[tid + 1] = incl_pull;
    if (tid == 0) sbase[0] = 0;
    if (tid == E - 1) p.scalars[1] = incl_pull;  // n_pull
    __syncthreads();
    for (int base = t0; base < t1; base += 64) {
        const int t = base + lane;
        int emin = E;
        if (t < t1)
            for (int j = 0; j < k; ++j) {
                const int e = local_expert(ids, (int64_t)t * k + j, begin, E);
                if (e >= 0 && e < emin) emin = e;
            }
        const bool valid = emin < E;
        const uint64_t peers = match_peers(valid, emin, nbits);
        if (valid) {
            const int rank = __popcll(peers & lanes_lt());
            const int cur = wcnt[w * E + emin];
            p.pull_order[sbase[emin] + cur + rank] = t;
            if (rank == 0) wcnt[w * E + emin] = cur + __popcll(peers);
        }
    }
}

}  // namespace

hipError_t launch_route(const moe_shape& s, const int64_t* topk_idx, const PlanPtrs& p, hipStream_t stream) {
    const int E = s.num_experts;
    const size_t lds = (size_t)(kWaves * E + (E + 1) + E + (E + 1) + 64) * sizeof(int32_t);
    hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kThreads), lds, stream, topk_idx, s.num_tokens, s.topk, E,
                       s.expert_begin, s.block_m, p);
    return hipGetLastError();
}

}  // namespace moe
