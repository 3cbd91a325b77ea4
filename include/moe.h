/*
 * moe.h -- C ABI of the MI355X (gfx950) fused MoE expert FFN library
 * (libmoe_mi355x.so).
 *
 * One GPU's share of a mixture-of-experts FFN forward, as described by the
 * DeepGEMM "MegaMoE" pages and the fused-MoE practice page:
 *   routing tables -> grouped Linear1 (FP8 E4M3 activations x FP4 E2M1
 *   weights, UE8M0 per-32 scales) -> SwiGLU x top-k weight -> FP8 requant
 *   -> grouped Linear2 -> FP32 top-k combine written as BF16.
 *
 * Conventions for every entry point:
 *  - Tensor arguments are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or keeps them.  Row-major, contiguous.
 *  - Pointers must be 16-byte aligned (topk_idx 8, topk_w 4); the workspace
 *    pointers 256-byte aligned.  Otherwise MOE_ERR_ALIGN.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    outputs are valid once the stream reaches the call.  No call blocks on
 *    the GPU.  Calls that share a workspace must not overlap in time.
 *  - Stream capture: no call allocates, synchronizes or enqueues a memset,
 *    so the enqueueing calls can be recorded into a HIP graph and the graph
 *    replayed (the practice page rebuilds its schedule tables from a
 *    captured graph and allocates every buffer once for that reason,
 *    sections 2 and 5);
 *    replays are calls like any other and must not overlap on one
 *    workspace.  Call once eagerly before capturing (the first call on a
 *    device queries its properties).
 *  - Validation happens on the host before anything is enqueued, in this
 *    order: NULL shape (MOE_ERR_NULL), shape limits (MOE_ERR_SHAPE), the
 *    declared weight layout of the calls that read weights
 *    (MOE_ERR_LAYOUT), NULL pointers (MOE_ERR_NULL), alignment
 *    (MOE_ERR_ALIGN), workspace size (MOE_ERR_WORKSPACE), device
 *    architecture (MOE_ERR_ARCH).  A failed kernel launch returns
 *    MOE_ERR_HIP.  num_tokens == 0 is a no-op returning MOE_OK.
 *  - Expert ids outside [expert_begin, expert_begin + num_experts) are not
 *    errors: those top-k entries are simply not computed on this GPU (the
 *    pages' "valid expert" test).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,
    MOE_ERR_SHAPE = -2,
    MOE_ERR_ALIGN = -3,
    MOE_ERR_WORKSPACE = -4,
    MOE_ERR_ARCH = -5,
    MOE_ERR_HIP = -6,
    MOE_ERR_LAYOUT = -7
};

/* Layout of the expert weights a call is given (moe_shape.weight_layout). */
enum moe_weight_layout {
    MOE_WEIGHTS_PLAIN = 0,  /* row-major as drawn: see "plain" under moe_forward */
    MOE_WEIGHTS_TILED = 1   /* the output of moe_prepare_weights */
};

/* Problem shape.  Limits (else MOE_ERR_SHAPE, or MOE_ERR_ALIGN for the
 * divisibility rules):
 *   num_tokens   T >= 0, T * topk < 2^30
 *   hidden       H > 0, multiple of 256 (Linear1 K-steps of 128 and
 *                Linear2 output tiles of 256 columns)
 *   intermediate I > 0, multiple of 128 (Linear1 emits 2I interleaved
 *                gate/up columns in tiles of 256; Linear2 K-steps of 128)
 *   num_experts  E local experts, 1..512
 *   expert_begin global id of local expert 0
 *   topk         k, 1..64
 *   block_m      rows per routing block, one of 16, 32, 64, 96, 128, 192
 *                (the walk-through's BLOCK_M candidates, section 7.1); each
 *                expert's rows are padded to a multiple of it.
 * Linear1 epilogue variants (reading notes, "activation clamp" and the
 * fast-math switch of the SwiGLU step; walk-through section 4.6):
 *   swiglu_limit 0: no clamp (the default).  > 0: before SwiGLU the BF16
 *                gate value is clamped from above, gate = min(gate, limit),
 *                and the up value on both sides, up = clamp(up, -limit,
 *                limit) (the pages' default limit is 10).  Must be finite.
 *   exact_silu   0: silu(g) = g * rcp(1 + exp2(-g log2 e)) with the
 *                hardware exp2 and reciprocal (the default; the pages'
 *                fast-math path).  1: g / (1 + expf(-g)) with the accurate
 *                library expf and IEEE division.
 * Weight layout:
 *   weight_layout  MOE_WEIGHTS_PLAIN or MOE_WEIGHTS_TILED (else
 *                MOE_ERR_SHAPE): the layout of the w1/w1_sf/w2/w2_sf the
 *                call is given.  The calls that read weights
 *                (moe_forward, moe_linear1, moe_linear2, moe_expert_ffn)
 *                take only MOE_WEIGHTS_TILED and return MOE_ERR_LAYOUT for
 *                MOE_WEIGHTS_PLAIN (so a zero-initialised shape is refused
 *                there until the caller states that it ran
 *                moe_prepare_weights); the other calls ignore the field.
 */
typedef struct moe_shape {
    int32_t num_tokens;
    int32_t hidden;
    int32_t intermediate;
    int32_t num_experts;
    int32_t expert_begin;
    int32_t topk;
    int32_t block_m;
    float swiglu_limit;
    int32_t exact_silu;
    int32_t weight_layout;
} moe_shape;

/* Worst-case padded row count of the routing layout ("pool capacity"):
 * align(T * k + E * (block_m - 1), block_m).  This is the SymmBuffer page's
 * pool formula (section 6.2) for one rank, with k in place of min(k, E) so
 * that a token that names one expert twice stays in bounds; the two agree
 * for k <= E.  Returns MOE_OK and writes *rows, or an error status. */
MOE_API int moe_capacity_rows(const moe_shape* shape, int64_t* rows);

/* Routing block heuristic (walk-through section 7.1, "BLOCK_M selection"):
 * the expected rows per expert, num_tokens * topk / num_experts, times the
 * pages' imbalance factor 2 is the target; the result is the smallest
 * candidate of the pages' ladder (16, 32, 64, 96, 128, 192) that is >= the
 * target, else 192.
 *   num_tokens   tokens whose top-k lists are routed (all ranks' tokens,
 *                num_tokens x num_ranks in the pages' formula), >= 0
 *   topk         k, 1..64
 *   num_experts  experts the ids are drawn from (all ranks' experts), >= 1
 * Host only.  Returns MOE_OK and writes *block_m, MOE_ERR_NULL, or
 * MOE_ERR_SHAPE for arguments out of range (num_tokens < 2^40). */
MOE_API int moe_suggest_block_m(int64_t num_tokens, int32_t topk, int32_t num_experts,
                int32_t* block_m);

/* How many GEMM launches moe_expert_ffn and moe_forward make for this
 * shape on the current device: *expert_ffn = 1 if moe_expert_ffn runs
 * Linear1 and Linear2 as one persistent launch (see there), 2 if it falls
 * back to moe_linear1 + moe_linear2; *forward = 1 if moe_forward runs
 * moe_expert_ffn as one launch, 2 if it runs moe_linear1 + moe_linear2.
 * moe_forward takes the one launch when moe_expert_ffn supports it and
 * Linear1 has at most 16 tiles per compute unit in the worst case (every
 * hit local), bounded by (cap / M + E) * (2I / 512) tiles, M = 16 for
 * block_m 16, else 128, cap as in moe_capacity_rows (integer division).  Host only (the
 * compute-unit count of the current device; 256 if there is none).
 * Returns MOE_OK, MOE_ERR_NULL or a shape error. */
MOE_API int moe_gemm_launches(const moe_shape* shape, int32_t* expert_ffn, int32_t* forward);

/* ---- routing tables ------------------------------------------------------
 * What is built follows the practice page's schedule tables (section 2) and
 * the MegaMoE dispatch counting (walk-through section 4.2, steps 1 and 3):
 * per-expert hit counts, each expert's row range padded to block_m, a slot
 * for every valid top-k entry (rows of one expert in ascending t*k+j
 * order), the inverse tables, per-block expert id and padding slack, and the
 * pull order (tokens with a hit, ascending by their smallest slot).
 * The tables are bit-identical for identical inputs. */

/* Bytes of the plan workspace for this shape. */
MOE_API int moe_plan_workspace_bytes(const moe_shape* shape, size_t* bytes);

/* Build the routing tables of topk_idx (int64 [T, k], global expert ids)
 * into plan_ws (>= moe_plan_workspace_bytes, 256-byte aligned), together
 * with the two grouped GEMMs' tile lists, which depend on the routing only.
 * One kernel launch (three for more than 4096 hits); nothing to initialise
 * beforehand. */
MOE_API int moe_plan(const moe_shape* shape, const int64_t* topk_idx,
             void* plan_ws, size_t plan_ws_bytes, void* stream);

/* Device pointers to the tables inside a plan workspace (no GPU work).
 *   scalars[4]      int32: R_pad (padded rows used), n_pull, N (valid hits),
 *                   n_blocks (= R_pad / block_m)
 *   counts[E]       hits per local expert
 *   offsets[E+1]    first padded row of each expert; offsets[E] = R_pad
 *   slot[T*k]       row of top-k entry (t, j), -1 if not local
 *   row_token[cap]  token of each row, -1 for padding (rows < R_pad)
 *   row_topk[cap]   top-k index j of each row, -1 for padding (rows < R_pad)
 *   block_expert[cap/block_m]  local expert of each block (blocks < n_blocks)
 *   slack[cap/block_m]         padding rows of each block (blocks < n_blocks)
 *   pull_order[T]   tokens with >= 1 local hit by smallest slot (first n_pull)
 * Entries past the stated ranges are unspecified. */
typedef struct moe_plan_view {
    int32_t* scalars;
    int32_t* counts;
    int32_t* offsets;
    int32_t* slot;
    int32_t* row_token;
    int32_t* row_topk;
    int32_t* block_expert;
    int32_t* slack;
    int32_t* pull_order;
    int64_t capacity_rows;
} moe_plan_view;
MOE_API int moe_plan_view_get(const moe_shape* shape, void* plan_ws, moe_plan_view* out);

/* ---- forward ---------------------------------------------------------------
 * Inputs (formats of the reading notes' "numerical formats" table):
 *   x        uint8 [T, H]        FP8 E4M3 (OCP, max 448)
 *   x_sf     uint8 [T, H/32]     UE8M0 scale of each 32 consecutive x values
 *   topk_idx int64 [T, k]        global expert ids
 *   topk_w   float [T, k]        routing weights (applied in the Linear1
 *                                epilogue, walk-through section 4.6)
 *   w1, w1_sf, w2, w2_sf         the expert weights in the TILED layout made
 *                                once by moe_prepare_weights (below) from the
 *                                plain layout; the shape must say so
 *                                (weight_layout = MOE_WEIGHTS_TILED), else
 *                                the call returns MOE_ERR_LAYOUT:
 *     plain w1    uint8 [E, 2I, H/2]  FP4 E2M1 pairs, even K in the low
 *                                     nibble; rows interleave gate/up by 8:
 *                                     [g0..7, u0..7, g8..15, u8..15, ...]
 *                                     (walk-through section 7.3)
 *     plain w1_sf uint8 [E, 2I, H/32] UE8M0, one per row per 32 K
 *     plain w2    uint8 [E, H, I/2]   FP4 E2M1 pairs
 *     plain w2_sf uint8 [E, H, I/32]  UE8M0
 * Output:
 *   y        uint16 [T, H]       BF16; y[t] = sum over t's local top-k
 *                                entries (j ascending, FP32) of the BF16
 *                                Linear2 rows; +0 for a token with none.
 * plan_ws: tables built by moe_plan for the same topk_idx and shape, or
 *   NULL to build them inside ws as part of this call.
 * ws: workspace of >= moe_forward_workspace_bytes, 256-byte aligned, any
 *   initial contents; holds the FP8 Linear2 input (and its scales), the BF16
 *   per-slot Linear2 rows between kernels, and the single launch's
 *   completion flags, launch counter and status word (see moe_expert_ffn).
 *   If the GEMMs ran as one launch and a Linear2 tile gave up waiting
 *   (see moe_expert_ffn), every element of y is NaN. */
MOE_API int moe_forward_workspace_bytes(const moe_shape* shape, size_t* bytes);

/* One-time weight re-layout (the analog of the pages' weight transform,
 * SymmBuffer page section 7: their forward also consumes weights prepared
 * once for the kernel).  which = 1: W1 (N = 2I rows, K = H); which = 2: W2
 * (N = H, K = I).  Reads the plain layout (w [E, N, K/2], w_sf [E, N, K/32])
 * and writes the tiled layout, a permutation of the same bytes (w_tiled has
 * E*N*K/2 bytes, w_sf_tiled E*N*K/32):
 *   w_tiled    [E][N/256][K/128][1024 slots of 16 B]: slot p holds bytes
 *              [kt*64 + q*16, +16) of tile column c = p >> 2, with
 *              q = (p & 3) ^ ((c >> 1) & 3);
 *   w_sf_tiled [E][N/256][K/128][256 columns][4 B]: the column's four
 *              scale bytes for that K-step;
 *   tile column c of block nt holds weight row nt*256 + src(c):
 *     which = 1 (c = 64G + 16b + j, b < 4, j < 16):
 *                src = 16*(ch/8) + ch%8 + (b >= 2 ? 8 : 0) with
 *                ch = 32G + 2j + b%2 (gate row of channel ch for
 *                b < 2, its up row otherwise);
 *     which = 2 (c = 128S + 16b + j, b < 8, j < 16): src = 128S + 8j + b.
 * Enqueued on `stream`; buffers owned by the caller; in and out must not
 * overlap. */
MOE_API int moe_prepare_weights(const moe_shape* shape, int which,
                const uint8_t* w, const uint8_t* w_sf,
                uint8_t* w_tiled, uint8_t* w_sf_tiled, void* stream);
MOE_API int moe_forward(const moe_shape* shape,
                const uint8_t* x, const uint8_t* x_sf,
                const int64_t* topk_idx, const float* topk_w,
                const uint8_t* w1, const uint8_t* w1_sf,
                const uint8_t* w2, const uint8_t* w2_sf,
                uint16_t* y,
                const void* plan_ws,
                void* ws, size_t ws_bytes, void* stream);

/* ---- the forward's stages (Linear1 gathers its rows, their scales and the
 * top-k weights through the plan's row tables itself) ------------------------
 * moe_forward(plan_ws != NULL) is exactly moe_expert_ffn or moe_linear1 then
 * moe_linear2 (the choice moe_gemm_launches reports), then moe_combine, in
 * this order on one stream (with plan_ws NULL its routing kernels also do
 * the single launch's one-thread prepare work, one kernel fewer); moe_expert_ffn computes what moe_linear1 then
 * moe_linear2 compute (bit for bit), in one persistent launch where the
 * shape allows it.  (With few Linear1 tiles per CU the single launch saves a
 * kernel tail and ramp; with many it measured slightly slower.)  They are
 * exposed so a caller can schedule or time the stages itself.  Arguments mean what they mean for moe_forward; plan_ws
 * (from moe_plan) is required here, and ws must be the same forward
 * workspace for all of them.  moe_linear1 clears the workspace's status word
 * (nothing in the two-launch schedule sets it).
 *   moe_linear1: grouped Linear1 over the routing layout with the fused
 *     SwiGLU x top-k weight and FP8 requant epilogue -> h_q, h_sf in ws
 *     (reading notes "stage three" and "stage four").
 *   moe_linear2: grouped Linear2 of h_q with BF16 output -> yslot in ws
 *     ("stage five").
 *   moe_combine: y[t] = BF16(FP32 sum over j of yslot[slot[t, j]])
 *     ("stage six"; walk-through section 4.6 "combine reduction"); NaN in
 *     every element of y instead when the status word is non-zero. */
MOE_API int moe_linear1(const moe_shape* shape,
                const uint8_t* x, const uint8_t* x_sf, const float* topk_w,
                const uint8_t* w1, const uint8_t* w1_sf,
                const void* plan_ws, void* ws, size_t ws_bytes, void* stream);
MOE_API int moe_linear2(const moe_shape* shape,
                const uint8_t* w2, const uint8_t* w2_sf,
                const void* plan_ws, void* ws, size_t ws_bytes, void* stream);
MOE_API int moe_combine(const moe_shape* shape, const void* plan_ws,
                const void* ws, size_t ws_bytes, uint16_t* y, void* stream);

/* Linear1 and Linear2 in one persistent launch: the single-launch schedule of
 * the reading notes (execution path, item 6, and "stage two": Linear2 blocks
 * wait on arrival marks set by the Linear1 epilogue; walk-through section
 * 4.3).  One workgroup per CU runs its Linear1 tiles, then its Linear2 tiles;
 * a Linear2 tile starts once every Linear1 tile of its rows has stored them.
 * Used when 2I and H are multiples of 512, both K-loops are long enough for
 * the persistent kernel (H/128 and I/128 >= 4 for block_m >= 32, >= 6 for
 * block_m 16) and 2I/512 <= 64; otherwise this is moe_linear1 + moe_linear2.
 * The completion flags live in ws (any initial contents).  Ahead of every
 * single launch, eager or recorded into a graph, a one-thread kernel
 * advances a launch counter in ws and clears the status word; the launch
 * stamps its flags with a value derived one-to-one from the counter, so no
 * two of 2^32 successive launches on one workspace stamp the same value and
 * a flag left by an earlier launch never reads as set.  Calls sharing a ws
 * must not overlap.  A Linear2 tile that waits for about half a second
 * gives up, sets the forward view's sync_status to 1 and computes on rows
 * that may be unfinished (the launch needs every workgroup resident at
 * once, e.g. no other kernel occupying compute units); moe_combine then
 * writes NaN over all of y.  The word reports on the latest GEMM launch on
 * the workspace: the single launch clears it first, moe_linear1 clears it. */
MOE_API int moe_expert_ffn(const moe_shape* shape,
                const uint8_t* x, const uint8_t* x_sf, const float* topk_w,
                const uint8_t* w1, const uint8_t* w1_sf,
                const uint8_t* w2, const uint8_t* w2_sf,
                const void* plan_ws, void* ws, size_t ws_bytes, void* stream);

/* Device pointers to the intermediates inside a forward workspace, for
 * tests (no GPU work):
 *   h_q   uint8  [cap, I]     FP8 E4M3 Linear2 input (SwiGLU x w, requantised)
 *   h_sf  uint8  [cap/block_m][I/128][block_m][4]  its UE8M0 scales: the
 *         scale of row r, 32-channel group g is at
 *         [r / block_m][g / 4][r % block_m][g % 4]
 *   yslot uint16 [cap, H]     BF16 Linear2 output per slot row
 *   plan  the plan region used when moe_forward got plan_ws == NULL
 *   sync_status  uint32 word: 1 if the latest single-launch GEMM on this
 *         workspace gave up waiting (see moe_expert_ffn), else 0 once any
 *         GEMM has run on the workspace
 * Rows of padding (and rows >= R_pad) hold unspecified values. */
typedef struct moe_forward_view {
    uint8_t* h_q;
    uint8_t* h_sf;
    uint16_t* yslot;
    void* plan;
    int64_t capacity_rows;
    uint32_t* sync_status;
} moe_forward_view;
MOE_API int moe_forward_view_get(const moe_shape* shape, void* ws, moe_forward_view* out);

/* ---- forward without a caller workspace -----------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture that must not call hipMalloc, tight serving loops, harnesses that
 * forbid allocation.  moe_forward_noalloc computes exactly what moe_forward
 * computes with plan_ws = NULL (the same kernels, bit for bit), but its
 * forward workspace (routing tables included) is a device array inside the
 * library of MOE_NOALLOC_WORKSPACE_BYTES bytes per GPU, which every GPU the
 * library runs it on holds until the process ends.  The caller passes only
 * inputs and outputs, with moe_forward's meaning, layout and alignment.
 *   - Shapes whose moe_forward_workspace_bytes exceeds
 *     MOE_NOALLOC_WORKSPACE_BYTES are refused with MOE_ERR_WORKSPACE before
 *     any GPU work (the decode-sized batches fit: 128 tokens, hidden 7168,
 *     intermediate 2048, 32 experts, top-8, block_m 16 needs ~25 MB).
 *   - No call allocates or frees device memory, and none enqueues a memset.
 *     The first call on a device resolves the array's address there (call
 *     once eagerly before capturing a graph).
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents; nothing in it must start at zero (tables are rebuilt,
 *     completion flags are stamped from a launch counter, the status word is
 *     cleared by every GEMM launch).  Calls that overlap in time on one GPU
 *     (different streams, or different host threads) race on the array and
 *     give undefined results: serialise them.
 * Validation as for moe_forward; MOE_ERR_HIP also if the array's address
 * cannot be resolved. */
#define MOE_NOALLOC_WORKSPACE_BYTES (32u << 20)
MOE_API int moe_forward_noalloc(const moe_shape* shape,
                const uint8_t* x, const uint8_t* x_sf,
                const int64_t* topk_idx, const float* topk_w,
                const uint8_t* w1, const uint8_t* w1_sf,
                const uint8_t* w2, const uint8_t* w2_sf,
                uint16_t* y, void* stream);

/* MOE_OK if `device` is a gfx950 GPU, MOE_ERR_ARCH if not, MOE_ERR_HIP if
 * the runtime cannot be queried. */
MOE_API int moe_device_supported(int device);

/* Static string naming a status code. */
MOE_API const char* moe_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
