// Internal declarations shared by the library's translation units: workspace
// layout, kernel launchers and small device helpers for gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/moe.h"

namespace moe {

constexpr int kMaxExperts = 512;
constexpr int kMaxTopk = 64;
constexpr size_t kAlign = 256;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Offsets (bytes) of each table inside a plan workspace.
// Routing of large inputs runs over groups of route_group_tokens(T) tokens: 64, or 128 or 256 when
// that keeps the groups to at most kRouteMaxGroups (each group of the fused scan reads the counts of
// all groups, so their number must stay small).  A group's four waves take a quarter each, at most
// one token per lane.
constexpr int kRouteMaxGroups = 256;
inline int route_group_tokens(int64_t num_tokens) {
    int tpg = 64;
    while (tpg < 256 && (num_tokens + tpg - 1) / tpg > kRouteMaxGroups) tpg *= 2;
    return tpg;
}

// Routing blocks (block_m) the library takes: the walk-through's BLOCK_M candidates (section 7.1).
constexpr int kBlockLadder[] = {16, 32, 64, 96, 128, 192};
constexpr int kBlockLadderSize = 6;
inline bool block_m_supported(int bm) {
    for (const int c : kBlockLadder)
        if (bm == c) return true;
    return false;
}

// Tile widths of the two GEMMs: 512 columns when N allows it, else 256.
inline int gemm_bn(int n) { return n % 512 == 0 ? 512 : 256; }
// GEMM M-tile: up to 128 rows of one expert once block_m >= 32 (several blocks, part of one, or, with
// blocks of 96 and 192 rows, spans that cross block boundaries: an expert's rows are cut into tiles of
// 128 from its first row up to its last hit, the last tile shorter, so no tile holds only padding);
// for smaller block_m (decode-sized batches, a block or two per expert) the tile is one block.
inline int gemm_bm(int block_m) { return block_m >= 32 ? 128 : block_m; }
// Rows past `cap` that the row tables reserve, so a 128-row tile starting at the last block reads
// allocated memory (the GEMMs mask every row past the tile's valid count).
constexpr int kRowSlack = 128;
// Words per tile-list entry: {first row, n << 16 | e, valid rows, M-tile index}; M-tiles are
// numbered expert by expert over both lists, so Linear1 tile (M-tile i, N-tile n) and the Linear2
// tiles of M-tile i can find each other.
constexpr int kTileWords = 4;

struct PlanLayout {
    int64_t cap = 0, max_blocks = 0, groups = 0;
    int bmg = 0;                           // GEMM M-tile rows
    int nt1 = 0, nt2 = 0;                  // N-tiles of Linear1 (N = 2I) and Linear2 (N = H)
    int64_t max_tiles1 = 0, max_tiles2 = 0;
    size_t scalars = 0, counts = 0, offsets = 0, slot = 0, row_token = 0, row_topk = 0,
           block_expert = 0, slack = 0, pull_order = 0, group_counts = 0, tiles1 = 0, tiles2 = 0, total = 0;
};

inline int64_t capacity_rows(const moe_shape& s) {
    const int64_t raw = (int64_t)s.num_tokens * s.topk + (int64_t)s.num_experts * (s.block_m - 1);
    return (raw + s.block_m - 1) / s.block_m * s.block_m;
}

// Upper bound on the GEMM M-tiles of a routing: expert e has ceil(count_e / bmg) <= ceil(padded_e / bmg)
// of them, so at most R_pad / bmg + E over all experts, R_pad <= cap.
inline int64_t max_m_tiles(const moe_shape& s) {
    return (capacity_rows(s) + gemm_bm(s.block_m) - 1) / gemm_bm(s.block_m) + s.num_experts;
}

inline PlanLayout plan_layout(const moe_shape& s) {
    PlanLayout L;
    L.cap = capacity_rows(s);
    L.max_blocks = L.cap / s.block_m;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, kAlign); return at; };
    L.scalars = take(16 * sizeof(int32_t));
    L.counts = take((size_t)s.num_experts * 4);
    L.offsets = take((size_t)(s.num_experts + 1) * 4);
    L.slot = take((size_t)s.num_tokens * s.topk * 4);
    L.row_token = take((size_t)(L.cap + kRowSlack) * 4);
    L.row_topk = take((size_t)(L.cap + kRowSlack) * 4);
    L.block_expert = take((size_t)L.max_blocks * 4);
    L.slack = take((size_t)L.max_blocks * 4);
    L.pull_order = take((size_t)s.num_tokens * 4);
    L.groups = (s.num_tokens + route_group_tokens(s.num_tokens) - 1) / route_group_tokens(s.num_tokens);
    L.group_counts = take((size_t)L.groups * s.num_experts * 2 * 4);  // hit and pull counts per group
    // GEMM tile lists: tile = (expert, M-tile, N-tile), M-tile by M-tile, all N-tiles of each
    L.bmg = gemm_bm(s.block_m);
    L.nt1 = 2 * s.intermediate / gemm_bn(2 * s.intermediate);
    L.nt2 = s.hidden / gemm_bn(s.hidden);
    L.max_tiles1 = max_m_tiles(s) * L.nt1;
    L.max_tiles2 = max_m_tiles(s) * L.nt2;
    L.tiles1 = take((size_t)L.max_tiles1 * kTileWords * 4);
    L.tiles2 = take((size_t)L.max_tiles2 * kTileWords * 4);
    L.total = o;
    return L;
}

// Offsets (bytes) inside a forward workspace: the plan region first.
struct ForwardLayout {
    PlanLayout plan;
    size_t plan_base = 0, h_q = 0, h_sf = 0, yslot = 0, flags = 0, status = 0, epoch = 0, total = 0;
};

inline ForwardLayout forward_layout(const moe_shape& s) {
    ForwardLayout F;
    F.plan = plan_layout(s);
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, kAlign); return at; };
    F.plan_base = take(F.plan.total);
    F.h_q = take((size_t)F.plan.cap * s.intermediate);
    F.h_sf = take((size_t)F.plan.cap * (s.intermediate / 32));
    F.yslot = take((size_t)F.plan.cap * s.hidden * 2);
    F.flags = take((size_t)F.plan.max_tiles1 * 4);  // one word per Linear1 tile (fused launch)
    F.status = take(4);
    F.epoch = take(4);  // launch counter, advanced ahead of every single-launch GEMM
    F.total = o;
    return F;
}

// scalars: [0] R_pad, [1] n_pull, [2] N, [3] n_blocks, [4] Linear1 tiles, [5] Linear2 tiles
struct PlanPtrs {
    int32_t *scalars, *counts, *offsets, *slot, *row_token, *row_topk, *block_expert, *slack, *pull_order,
        *group_counts, *tiles1, *tiles2;
    int nt1, nt2, bmg;
    // Optional: when set, the routing kernels also do the single launch's prepare work (advance the
    // workspace's launch counter, clear its status word), so that a single launch enqueued right after
    // them needs no prepare kernel of its own (moe_forward building its plan inside the workspace).
    uint32_t* epoch_word = nullptr;
    uint32_t* status = nullptr;
};

inline PlanPtrs plan_ptrs(const PlanLayout& L, void* base) {
    char* b = static_cast<char*>(base);
    auto at = [&](size_t off) { return reinterpret_cast<int32_t*>(b + off); };
    PlanPtrs p;
    p.scalars = at(L.scalars); p.counts = at(L.counts); p.offsets = at(L.offsets); p.slot = at(L.slot);
    p.row_token = at(L.row_token); p.row_topk = at(L.row_topk); p.block_expert = at(L.block_expert);
    p.slack = at(L.slack); p.pull_order = at(L.pull_order); p.group_counts = at(L.group_counts);
    p.tiles1 = at(L.tiles1); p.tiles2 = at(L.tiles2);
    p.nt1 = L.nt1; p.nt2 = L.nt2; p.bmg = L.bmg;
    return p;
}

// ---- launchers (each enqueues on `stream` and returns the launch status) ----
hipError_t launch_route(const moe_shape& s, const int64_t* topk_idx, const PlanPtrs& p, hipStream_t stream);

struct GemmProblem {
    const moe_shape* shape;
    const PlanPtrs* plan;
    int64_t cap;
};
// Linear1 gathers its A rows and their scales (x [T, H], x_sf [T, H/32]) and
// the top-k weights through the plan's row tables; Linear2 reads h_q and h_sf
// (per-block layout [cap/bm][I/128][bm][4]) as the Linear1 epilogue wrote
// them.  w*, w*_sf: weights in the tiled layout of moe_prepare.hip.
// status: the forward's status word, cleared by the Linear1 launch (nothing in the two-launch schedule
// sets it).
hipError_t launch_linear1(const GemmProblem& g, const uint8_t* x, const uint8_t* x_sf, const float* topk_w,
                          const uint8_t* w1, const uint8_t* w1_sf, uint8_t* h_q, uint8_t* h_sf, uint32_t* status,
                          hipStream_t stream);
hipError_t launch_linear2(const GemmProblem& g, const uint8_t* h_q, const uint8_t* h_sf, const uint8_t* w2,
                          const uint8_t* w2_sf, uint16_t* yslot, hipStream_t stream);
// Both GEMMs in one persistent launch when the shape allows it (fused_supported), else the two
// launches above.  flags: one word per Linear1 tile, any initial contents; status: cleared ahead of the
// launch, set to 1 if a Linear2 tile stopped waiting for its rows; epoch_word: the workspace's launch
// counter (any initial contents), advanced by a one-thread kernel ahead of every single launch.
bool fused_supported(const moe_shape& s);
// moe_forward runs both GEMMs as that one launch while Linear1 has at most kOneLaunchTilesPerCu tiles
// per CU in the worst case (every hit local), else as two launches: the single launch hides the
// first launch's tail and the second one's ramp, which matter only while there are few tiles per CU,
// and its per-tile cost is a little higher (device-coherent stores, flag polls).
constexpr int kOneLaunchTilesPerCu = 16;
bool forward_one_launch(const moe_shape& s, int cus);
int cu_count();  // compute units of the current device (256 if it cannot be queried)
// prepared: the kernels enqueued just before this call did the prepare work already (PlanPtrs'
// epoch_word and status), so no prepare kernel is enqueued.
hipError_t launch_expert_ffn(const GemmProblem& g, const uint8_t* x, const uint8_t* x_sf, const float* topk_w,
                             const uint8_t* w1, const uint8_t* w1_sf, uint8_t* h_q, uint8_t* h_sf,
                             const uint8_t* w2, const uint8_t* w2_sf, uint16_t* yslot, uint32_t* flags,
                             uint32_t* status, uint32_t* epoch_word, hipStream_t stream, bool prepared = false);
hipError_t launch_tile_weights(int which, int N, int K, int E, const uint8_t* w, const uint8_t* w_sf,
                               uint8_t* w_out, uint8_t* sf_out, hipStream_t stream);
// status: the forward's status word; when it is non-zero (a single-launch GEMM gave up waiting) every
// element of y is written as NaN.
hipError_t launch_combine(const moe_shape& s, const uint16_t* yslot, const int32_t* slot, const uint32_t* status,
                          uint16_t* y, hipStream_t stream);

}  // namespace moe
