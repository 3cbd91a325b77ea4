// C ABI of the fused MoE expert FFN library: host-side validation,
// workspace carving and the kernel sequence
//   routing -> Linear1 (+SwiGLU/requant) -> Linear2 (+BF16) -> combine,
// all enqueued on the caller's stream.  Interface modelled on the pages'
// host API: a size query plus caller-owned buffer (SymmBuffer page,
// sections 5-6), one forward entry point with strict shape checks that
// answer "unsupported" (reading notes, "host-side checks").
#include <atomic>
#include <cstring>
#include <mutex>

#include "moe_internal.h"

using namespace moe;

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture
std::atomic<int> g_arch_cache[kMaxDevices];

int check_arch_current() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    return moe_device_supported(dev);
}

int check_shape(const moe_shape* s) {
    if (!s) return MOE_ERR_NULL;
    if (s->num_tokens < 0 || s->hidden <= 0 || s->intermediate <= 0) return MOE_ERR_SHAPE;
    if (s->num_experts < 1 || s->num_experts > kMaxExperts) return MOE_ERR_SHAPE;
    if (s->topk < 1 || s->topk > kMaxTopk) return MOE_ERR_SHAPE;
    if (!block_m_supported(s->block_m)) return MOE_ERR_SHAPE;
    if ((int64_t)s->num_tokens * s->topk >= (1ll << 30)) return MOE_ERR_SHAPE;
    if (!(s->swiglu_limit >= 0.0f && s->swiglu_limit <= 3.0e38f)) return MOE_ERR_SHAPE;  // also rejects NaN
    if (s->exact_silu != 0 && s->exact_silu != 1) return MOE_ERR_SHAPE;
    if (s->weight_layout != MOE_WEIGHTS_PLAIN && s->weight_layout != MOE_WEIGHTS_TILED) return MOE_ERR_SHAPE;
    if (s->hidden > (1 << 20) || s->intermediate > (1 << 20)) return MOE_ERR_SHAPE;
    if (s->hidden % 256 != 0 || s->intermediate % 128 != 0) return MOE_ERR_ALIGN;
    // kernels address each operand's rows with 32-bit offsets
    const int64_t lim = 1ll << 31;
    if ((int64_t)s->num_tokens * s->hidden >= lim) return MOE_ERR_SHAPE;
    if (capacity_rows(*s) * s->intermediate >= lim) return MOE_ERR_SHAPE;
    if ((int64_t)s->hidden * s->intermediate >= lim) return MOE_ERR_SHAPE;
    return MOE_OK;
}

// The calls that read weights: a valid shape that also declares the tiled layout.
int check_weight_shape(const moe_shape* s) {
    const int st = check_shape(s);
    if (st != MOE_OK) return st;
    return s->weight_layout == MOE_WEIGHTS_TILED ? MOE_OK : MOE_ERR_LAYOUT;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

int moe_device_supported(int device) {
    if (device < 0) return MOE_ERR_HIP;
    if (device < kMaxDevices) {
        const int c = g_arch_cache[device].load(std::memory_order_relaxed);
        if (c == 1) return MOE_OK;
        if (c == 2) return MOE_ERR_ARCH;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return MOE_ERR_HIP;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (device < kMaxDevices) g_arch_cache[device].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? MOE_OK : MOE_ERR_ARCH;
}

const char* moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "null pointer";
        case MOE_ERR_SHAPE: return "unsupported shape";
        case MOE_ERR_ALIGN: return "misaligned pointer or dimension";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_ARCH: return "device is not gfx950";
        case MOE_ERR_HIP: return "HIP runtime error";
        case MOE_ERR_LAYOUT: return "weights not declared in the tiled layout";
        default: return "unknown status";
    }
}

int moe_capacity_rows(const moe_shape* shape, int64_t* rows) {
    if (!rows) return MOE_ERR_NULL;
    const int st = check_shape(shape);
    if (st != MOE_OK) return st;
    *rows = capacity_rows(*shape);
    return MOE_OK;
}

int moe_suggest_block_m(int64_t num_tokens, int32_t topk, int32_t num_experts, int32_t* block_m) {
    if (!block_m) return MOE_ERR_NULL;
    if (num_tokens < 0 || num_tokens >= (1ll << 40) || topk < 1 || topk > kMaxTopk || num_experts < 1)
        return MOE_ERR_SHAPE;
    // target rows = imbalance factor 2 x expected rows per expert (T * k / E); the smallest routing
    // block of the pages' ladder that holds the target, compared exactly in integers: 2 T k <= c E
    const int64_t twice_hits = 2 * num_tokens * topk;
    int32_t pick = kBlockLadder[kBlockLadderSize - 1];
    for (const int32_t c : kBlockLadder)
        if (twice_hits <= (int64_t)c * num_experts) {
            pick = c;
            break;
        }
    *block_m = pick;
    return MOE_OK;
}

int moe_gemm_launches(const moe_shape* shape, int32_t* expert_ffn, int32_t* forward) {
    if (!expert_ffn || !forward) return MOE_ERR_NULL;
    const int st = check_shape(shape);
    if (st != MOE_OK) return st;
    *expert_ffn = fused_supported(*shape) ? 1 : 2;
    *forward = forward_one_launch(*shape, cu_count()) ? 1 : 2;
    return MOE_OK;
}

int moe_plan_workspace_bytes(const moe_shape* shape, size_t* bytes) {
    if (!bytes) return MOE_ERR_NULL;
    const int st = check_shape(shape);
    if (st != MOE_OK) return st;
    *bytes = plan_layout(*shape).total;
    return MOE_OK;
}

int moe_forward_workspace_bytes(const moe_shape* shape, size_t* bytes) {
    if (!bytes) return MOE_ERR_NULL;
    const int st = check_shape(shape);
    if (st != MOE_OK) return st;
    *bytes = forward_layout(*shape).total;
    return MOE_OK;
}

int moe_plan_view_get(const moe_shape* shape, void* plan_ws, moe_plan_view* out) {
    if (!out || !plan_ws) return MOE_ERR_NULL;
    const int st = check_shape(shape);
    if (st != MOE_OK) return st;
    const PlanLayout L = plan_layout(*shape);
    const PlanPtrs p = plan_ptrs(L, plan_ws);
    out->scalars = p.scalars; out->counts = p.counts; out->offsets = p.offsets; out->slot = p.slot;
    out->row_token = p.row_token; out->row_topk = p.row_topk; out->block_expert = p.block_expert;
    out->slack = p.slack; out->pull_order = p.pull_order; out->capacity_rows = L.cap;
    return MOE_OK;
}

int moe_forward_view_get(const moe_shape* shape, void* ws, moe_forward_view* out) {
    if (!out || !ws) return MOE_ERR_NULL;
    const int st = check_shape(shape);
    if (st != MOE_OK) return st;
    const ForwardLayout F = forward_layout(*shape);
    char* b = static_cast<char*>(ws);
    out->h_q = reinterpret_cast<uint8_t*>(b + F.h_q);
    out->h_sf = reinterpret_cast<uint8_t*>(b + F.h_sf);
    out->yslot = reinterpret_cast<uint16_t*>(b + F.yslot);
    out->plan = b + F.plan_base;
    out->capacity_rows = F.plan.cap;
    out->sync_status = reinterpret_cast<uint32_t*>(b + F.status);
    return MOE_OK;
}

int moe_plan(const moe_shape* shape, const int64_t* topk_idx, void* plan_ws, size_t plan_ws_bytes,
             void* stream) {
    int st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->num_tokens == 0) return MOE_OK;
    if (!topk_idx || !plan_ws) return MOE_ERR_NULL;
    if (!aligned(topk_idx, 8) || !aligned(plan_ws, kAlign)) return MOE_ERR_ALIGN;
    const PlanLayout L = plan_layout(*shape);
    if (plan_ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    if ((st = check_arch_current()) != MOE_OK) return st;
    const hipError_t e = launch_route(*shape, topk_idx, plan_ptrs(L, plan_ws), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_prepare_weights(const moe_shape* shape, int which, const uint8_t* w, const uint8_t* w_sf, uint8_t* w_tiled,
                        uint8_t* w_sf_tiled, void* stream) {
    int st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (which != 1 && which != 2) return MOE_ERR_SHAPE;
    if (!w || !w_sf || !w_tiled || !w_sf_tiled) return MOE_ERR_NULL;
    if (!aligned(w, 16) || !aligned(w_tiled, 16) || !aligned(w_sf, 4) || !aligned(w_sf_tiled, 4))
        return MOE_ERR_ALIGN;
    if ((st = check_arch_current()) != MOE_OK) return st;
    const int N = which == 1 ? 2 * shape->intermediate : shape->hidden;
    const int K = which == 1 ? shape->hidden : shape->intermediate;
    const hipError_t e = launch_tile_weights(which, N, K, shape->num_experts, w, w_sf, w_tiled, w_sf_tiled,
                                             static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_linear1(const moe_shape* shape, const uint8_t* x, const uint8_t* x_sf, const float* topk_w,
                const uint8_t* w1, const uint8_t* w1_sf, const void* plan_ws, void* ws, size_t ws_bytes,
                void* stream) {
    int st = check_weight_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->num_tokens == 0) return MOE_OK;
    if (!x || !x_sf || !topk_w || !w1 || !w1_sf || !plan_ws || !ws) return MOE_ERR_NULL;
    if (!aligned(x, 16) || !aligned(x_sf, 16) || !aligned(w1, 16) || !aligned(w1_sf, 16) || !aligned(topk_w, 4) ||
        !aligned(ws, kAlign) || !aligned(plan_ws, kAlign))
        return MOE_ERR_ALIGN;
    const ForwardLayout F = forward_layout(*shape);
    if (ws_bytes < F.total) return MOE_ERR_WORKSPACE;
    if ((st = check_arch_current()) != MOE_OK) return st;
    const PlanPtrs p = plan_ptrs(F.plan, const_cast<void*>(plan_ws));
    char* base = static_cast<char*>(ws);
    const GemmProblem g{shape, &p, F.plan.cap};
    const hipError_t e = launch_linear1(g, x, x_sf, topk_w, w1, w1_sf, reinterpret_cast<uint8_t*>(base + F.h_q),
                                        reinterpret_cast<uint8_t*>(base + F.h_sf),
                                        reinterpret_cast<uint32_t*>(base + F.status), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_linear2(const moe_shape* shape, const uint8_t* w2, const uint8_t* w2_sf, const void* plan_ws, void* ws,
                size_t ws_bytes, void* stream) {
    int st = check_weight_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->num_tokens == 0) return MOE_OK;
    if (!w2 || !w2_sf || !plan_ws || !ws) return MOE_ERR_NULL;
    if (!aligned(w2, 16) || !aligned(w2_sf, 16) || !aligned(ws, kAlign) || !aligned(plan_ws, kAlign))
        return MOE_ERR_ALIGN;
    const ForwardLayout F = forward_layout(*shape);
    if (ws_bytes < F.total) return MOE_ERR_WORKSPACE;
    if ((st = check_arch_current()) != MOE_OK) return st;
    const PlanPtrs p = plan_ptrs(F.plan, const_cast<void*>(plan_ws));
    char* base = static_cast<char*>(ws);
    const GemmProblem g{shape, &p, F.plan.cap};
    const hipError_t e = launch_linear2(g, reinterpret_cast<uint8_t*>(base + F.h_q),
                                        reinterpret_cast<uint8_t*>(base + F.h_sf), w2, w2_sf,
                                        reinterpret_cast<uint16_t*>(base + F.yslot), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"

namespace {
// moe_expert_ffn; prepared: the routing kernels enqueued just before did the single launch's prepare
// work (moe_forward building its plan inside ws), so no prepare kernel is enqueued.
int expert_ffn_call(const moe_shape* shape, const uint8_t* x, const uint8_t* x_sf, const float* topk_w,
                    const uint8_t* w1, const uint8_t* w1_sf, const uint8_t* w2, const uint8_t* w2_sf,
                    const void* plan_ws, void* ws, size_t ws_bytes, void* stream, bool prepared) {
    int st = check_weight_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->num_tokens == 0) return MOE_OK;
    if (!x || !x_sf || !topk_w || !w1 || !w1_sf || !w2 || !w2_sf || !plan_ws || !ws) return MOE_ERR_NULL;
    if (!aligned(x, 16) || !aligned(x_sf, 16) || !aligned(w1, 16) || !aligned(w1_sf, 16) || !aligned(w2, 16) ||
        !aligned(w2_sf, 16) || !aligned(topk_w, 4) || !aligned(ws, kAlign) || !aligned(plan_ws, kAlign))
        return MOE_ERR_ALIGN;
    const ForwardLayout F = forward_layout(*shape);
    if (ws_bytes < F.total) return MOE_ERR_WORKSPACE;
    if ((st = check_arch_current()) != MOE_OK) return st;
    const PlanPtrs p = plan_ptrs(F.plan, const_cast<void*>(plan_ws));
    char* base = static_cast<char*>(ws);
    const GemmProblem g{shape, &p, F.plan.cap};
    const hipError_t e = launch_expert_ffn(
        g, x, x_sf, topk_w, w1, w1_sf, reinterpret_cast<uint8_t*>(base + F.h_q),
        reinterpret_cast<uint8_t*>(base + F.h_sf), w2, w2_sf, reinterpret_cast<uint16_t*>(base + F.yslot),
        reinterpret_cast<uint32_t*>(base + F.flags), reinterpret_cast<uint32_t*>(base + F.status),
        reinterpret_cast<uint32_t*>(base + F.epoch), static_cast<hipStream_t>(stream), prepared);
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
}  // namespace

extern "C" {

int moe_expert_ffn(const moe_shape* shape, const uint8_t* x, const uint8_t* x_sf, const float* topk_w,
                   const uint8_t* w1, const uint8_t* w1_sf, const uint8_t* w2, const uint8_t* w2_sf,
                   const void* plan_ws, void* ws, size_t ws_bytes, void* stream) {
    return expert_ffn_call(shape, x, x_sf, topk_w, w1, w1_sf, w2, w2_sf, plan_ws, ws, ws_bytes, stream, false);
}

int moe_combine(const moe_shape* shape, const void* plan_ws, const void* ws, size_t ws_bytes, uint16_t* y,
                void* stream) {
    int st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->num_tokens == 0) return MOE_OK;
    if (!plan_ws || !ws || !y) return MOE_ERR_NULL;
    if (!aligned(y, 16) || !aligned(ws, kAlign) || !aligned(plan_ws, kAlign)) return MOE_ERR_ALIGN;
    const ForwardLayout F = forward_layout(*shape);
    if (ws_bytes < F.total) return MOE_ERR_WORKSPACE;
    if ((st = check_arch_current()) != MOE_OK) return st;
    const PlanPtrs p = plan_ptrs(F.plan, const_cast<void*>(plan_ws));
    const char* base = static_cast<const char*>(ws);
    const hipError_t e = launch_combine(*shape, reinterpret_cast<const uint16_t*>(base + F.yslot), p.slot,
                                        reinterpret_cast<const uint32_t*>(base + F.status), y,
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_forward(const moe_shape* shape, const uint8_t* x, const uint8_t* x_sf, const int64_t* topk_idx,
                const float* topk_w, const uint8_t* w1, const uint8_t* w1_sf, const uint8_t* w2,
                const uint8_t* w2_sf, uint16_t* y, const void* plan_ws, void* ws, size_t ws_bytes,
                void* stream) {
    int st = check_weight_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->num_tokens == 0) return MOE_OK;
    if (!x || !x_sf || !topk_idx || !topk_w || !w1 || !w1_sf || !w2 || !w2_sf || !y || !ws) return MOE_ERR_NULL;
    if (!aligned(x, 16) || !aligned(x_sf, 16) || !aligned(w1, 16) || !aligned(w1_sf, 16) || !aligned(w2, 16) ||
        !aligned(w2_sf, 16) || !aligned(y, 16) || !aligned(topk_idx, 8) || !aligned(topk_w, 4) ||
        !aligned(ws, kAlign) || (plan_ws && !aligned(plan_ws, kAlign)))
        return MOE_ERR_ALIGN;
    const ForwardLayout F = forward_layout(*shape);
    if (ws_bytes < F.total) return MOE_ERR_WORKSPACE;
    if ((st = check_arch_current()) != MOE_OK) return st;
    char* base = static_cast<char*>(ws);
    const void* plan = plan_ws ? plan_ws : static_cast<const void*>(base + F.plan_base);
    const bool one_launch = forward_one_launch(*shape, cu_count());
    if (!plan_ws) {
        PlanPtrs pp = plan_ptrs(F.plan, base + F.plan_base);
        if (one_launch) {  // the routing kernels also do the single launch's prepare work
            pp.epoch_word = reinterpret_cast<uint32_t*>(base + F.epoch);
            pp.status = reinterpret_cast<uint32_t*>(base + F.status);
        }
        const hipError_t e = launch_route(*shape, topk_idx, pp, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    if (one_launch) {
        if ((st = expert_ffn_call(shape, x, x_sf, topk_w, w1, w1_sf, w2, w2_sf, plan, ws, ws_bytes, stream,
                                  !plan_ws)) != MOE_OK)
            return st;
    } else {
        if ((st = moe_linear1(shape, x, x_sf, topk_w, w1, w1_sf, plan, ws, ws_bytes, stream)) != MOE_OK) return st;
        if ((st = moe_linear2(shape, w2, w2_sf, plan, ws, ws_bytes, stream)) != MOE_OK) return st;
    }
    return moe_combine(shape, plan, ws, ws_bytes, y, stream);
}

// ---- allocation-free forward (moe_forward_noalloc)
// Its workspace is this file-scope device array: one copy per GPU, held until the process ends.  In
// host code the name `scratch` is only a host-side stand-in; the array's device address on a GPU comes
// from hipGetSymbolAddress, called once per device with that device current, and only that address is
// ever passed to kernels.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_WORKSPACE_BYTES];

}  // extern "C"

namespace {

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (resolved on the first call on that device).
int scratch_of_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward_noalloc(const moe_shape* shape, const uint8_t* x, const uint8_t* x_sf, const int64_t* topk_idx,
                        const float* topk_w, const uint8_t* w1, const uint8_t* w1_sf, const uint8_t* w2,
                        const uint8_t* w2_sf, uint16_t* y, void* stream) {
    int st = check_weight_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->num_tokens == 0) return MOE_OK;
    if (!x || !x_sf || !topk_idx || !topk_w || !w1 || !w1_sf || !w2 || !w2_sf || !y) return MOE_ERR_NULL;
    if (!aligned(x, 16) || !aligned(x_sf, 16) || !aligned(w1, 16) || !aligned(w1_sf, 16) || !aligned(w2, 16) ||
        !aligned(w2_sf, 16) || !aligned(y, 16) || !aligned(topk_idx, 8) || !aligned(topk_w, 4))
        return MOE_ERR_ALIGN;
    if (forward_layout(*shape).total > (size_t)MOE_NOALLOC_WORKSPACE_BYTES) return MOE_ERR_WORKSPACE;
    if ((st = check_arch_current()) != MOE_OK) return st;
    void* ws = nullptr;
    if ((st = scratch_of_current_device(&ws)) != MOE_OK) return st;
    // the routing tables go to the plan region of the workspace (plan_ws = NULL)
    return moe_forward(shape, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y, nullptr, ws,
                       (size_t)MOE_NOALLOC_WORKSPACE_BYTES, stream);
}

}  // extern "C"
