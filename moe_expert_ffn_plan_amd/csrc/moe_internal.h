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
// Routing of large inputs runs as three kernels over groups of kRouteTokensPerGroup tokens.
constexpr int kRouteTokensPerGroup = 256;

struct PlanLayout {
    int64_t cap = 0, max_blocks = 0, groups = 0;
    size_t scalars = 0, counts = 0, offsets = 0, slot = 0, row_token = 0, row_topk = 0,
           block_expert = 0, slack = 0, pull_order = 0, group_counts = 0, total = 0;
};

inline int64_t capacity_rows(const moe_shape& s) {
    const int64_t raw = (int64_t)s.num_tokens * s.topk + (int64_t)s.num_experts * (s.block_m - 1);
    return (raw + s.block_m - 1) / s.block_m * s.block_m;
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
    L.row_token = take((size_t)L.cap * 4);
    L.row_topk = take((size_t)L.cap * 4);
    L.block_expert = take((size_t)L.max_blocks * 4);
    L.slack = take((size_t)L.max_blocks * 4);
    L.pull_order = take((size_t)s.num_tokens * 4);
    L.groups = (s.num_tokens + kRouteTokensPerGroup - 1) / kRouteTokensPerGroup;
    L.group_counts = take((size_t)L.groups * s.num_experts * 2 * 4);  // hit and pull counts per group
    L.total = o;
    return L;
}

// Offsets (bytes) inside a forward workspace: the plan region first.
struct ForwardLayout {
    PlanLayout plan;
    size_t plan_base = 0, x_sf = 0, row_w = 0, tiles1 = 0, tiles2 = 0, h_q = 0, h_sf = 0, yslot = 0, total = 0;
    int64_t max_tiles1 = 0, max_tiles2 = 0;
};

// Tile widths of the two GEMMs: 512 columns when N allows it, else 256.
inline int gemm_bn(int n) { return n % 512 == 0 ? 512 : 256; }

inline ForwardLayout forward_layout(const moe_shape& s) {
    ForwardLayout F;
    F.plan = plan_layout(s);
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, kAlign); return at; };
    F.plan_base = take(F.plan.total);
    F.x_sf = take((size_t)F.plan.cap * (s.hidden / 32));
    F.row_w = take((size_t)F.plan.cap * 4);
    F.max_tiles1 = F.plan.max_blocks * (2 * s.intermediate / gemm_bn(2 * s.intermediate));
    F.max_tiles2 = F.plan.max_blocks * (s.hidden / gemm_bn(s.hidden));
    F.tiles1 = take((size_t)F.max_tiles1 * 8);
    F.tiles2 = take((size_t)F.max_tiles2 * 8);
    F.h_q = take((size_t)F.plan.cap * s.intermediate);
    F.h_sf = take((size_t)F.plan.cap * (s.intermediate / 32));
    F.yslot = take((size_t)F.plan.cap * s.hidden * 2);
    F.total = o;
    return F;
}

struct PlanPtrs {
    int32_t *scalars, *counts, *offsets, *slot, *row_token, *row_topk, *block_expert, *slack, *pull_order,
        *group_counts;
};

inline PlanPtrs plan_ptrs(const PlanLayout& L, void* base) {
    char* b = static_cast<char*>(base);
    return PlanPtrs{reinterpret_cast<int32_t*>(b + L.scalars),      reinterpret_cast<int32_t*>(b + L.counts),
                    reinterpret_cast<int32_t*>(b + L.offsets),      reinterpret_cast<int32_t*>(b + L.slot),
                    reinterpret_cast<int32_t*>(b + L.row_token),    reinterpret_cast<int32_t*>(b + L.row_topk),
                    reinterpret_cast<int32_t*>(b + L.block_expert), reinterpret_cast<int32_t*>(b + L.slack),
                    reinterpret_cast<int32_t*>(b + L.pull_order), reinterpret_cast<int32_t*>(b + L.group_counts)};
}

// ---- launchers (each enqueues on `stream` and returns the launch status) ----
hipError_t launch_route(const moe_shape& s, const int64_t* topk_idx, const PlanPtrs& p, hipStream_t stream);

struct GemmProblem {
    const moe_shape* shape;
    const PlanPtrs* plan;
    int64_t cap;
    const int32_t* tiles;  // tile list of this GEMM (written by the Linear1 prep kernel)
    const float* row_w;    // per-row top-k weights (Linear1 only)
};
// x_sf_tiled / h_sf: activation scales in the per-row-block layout [cap/BM][K/128][BM][4];
// w*, w*_sf: weights in the tiled layout of moe_prepare.hip.
hipError_t launch_linear1(const GemmProblem& g, const uint8_t* x, const uint8_t* x_sf_tiled,
                          const uint8_t* w1, const uint8_t* w1_sf, uint8_t* h_q, uint8_t* h_sf,
                          hipStream_t stream);
hipError_t launch_linear2(const GemmProblem& g, const uint8_t* h_q, const uint8_t* h_sf, const uint8_t* w2,
                          const uint8_t* w2_sf, uint16_t* yslot, hipStream_t stream);
hipError_t launch_tile_weights(int which, int N, int K, int E, const uint8_t* w, const uint8_t* w_sf,
                               uint8_t* w_out, uint8_t* sf_out, hipStream_t stream);
hipError_t launch_prep_linear1(const moe_shape& s, const uint8_t* x_sf, const float* topk_w, const PlanPtrs& p,
                               int64_t cap, int nt1, int nt2, uint32_t* xsf_out, float* row_w, int32_t* tiles1,
                               int32_t* tiles2, hipStream_t stream);
hipError_t launch_combine(const moe_shape& s, const uint16_t* yslot, const int32_t* slot, uint16_t* y,
                          hipStream_t stream);

}  // namespace moe
