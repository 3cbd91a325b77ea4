// Grouped FP8 x FP4 GEMMs of the MoE expert FFN on gfx950 scaled MFMA.
//
// Linear1: Z = X_e W1_e^T over each expert's padded row range (reading
// notes, "stage three": W1_e is [2*d_ff, d_model]); A rows are gathered from
// x through the routing table's row_token (no permuted copy of x).  Its
// epilogue rounds gate and up to BF16, applies SwiGLU and the top-k weight,
// takes the per-row 32-channel amax, picks the UE8M0 scale and writes FP8
// E4M3 codes (walk-through section 4.6; reading notes "stage four").
// Linear2: Y = H_e W2_e^T (W2_e is [d_model, d_ff]) on the requantised rows,
// FP32 accumulators rounded to BF16 (reading notes "stage five").
//
// Hardware mapping (CDNA4):
//  * V_MFMA_SCALE_F32_16X16X128_F8F6F4 with A = E4M3 and B = E2M1, the
//    UE8M0 block scales fed per lane.  Operand layout (measured on the
//    device): for A, lane l holds row l%16 and, for g = l/16, K bytes
//    [16g, 16g+16) in its first four dwords and [64+16g, 64+16g+16) in the
//    next four; the scale of (row r, K-group q) is taken from lane 16q + r.
//    For B (FP4), lane l holds column l%16 and K [32g, 32g+32) as 16 bytes,
//    even K in the low nibble, with its own lane's scale.  D: lane l holds
//    column l%16, rows 4(l/16)..4(l/16)+3.
//  * Workgroup = 4 waves (256 threads), tile BM x 256; wave w owns columns
//    [64w, 64w+64) of the tile, so every 64-column slice (32 gate/up
//    channels = one requant scale group) is reduced inside one wave.
//  * A (activations) is staged through LDS in 128-byte K-steps, double
//    buffered, 16-byte chunks XOR-swizzled by row so the MFMA-pattern reads
//    are bank-conflict free.  B (weights) is not shared between waves, so
//    each wave loads its own columns straight into registers one K-step
//    ahead.
//  * Tiles are listed expert by expert (for each N-tile, all M-tiles of the
//    expert) and blockIdx is remapped so that each XCD (blockIdx % 8 on
//    MI300-class parts) runs a contiguous run of that list: the M-tiles
//    sharing a weight tile run together on one XCD and hit its L2.
#include "moe_internal.h"

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBN = 256;
constexpr int kBK = 128;
constexpr int kNumXcd = 8;

struct GemmArgs {
    const uint8_t* a;      // Linear1: x [T, K]; Linear2: h_q [cap, K]
    const uint8_t* a_sf;   // [rows, K/32]
    const uint8_t* b;      // [E, N, K/2]
    const uint8_t* b_sf;   // [E, N, K/32]
    const int32_t* scalars;
    const int32_t* offsets;
    const int32_t* row_token;
    const int32_t* row_topk;
    const float* topk_w;
    uint8_t* out_q;        // Linear1: [cap, N/2]
    uint8_t* out_sf;       // Linear1: [cap, N/64]
    uint16_t* out_bf16;    // Linear2: [cap, N]
    int K, N, E, topk;
};

template <int BM>
__device__ __forceinline__ bool map_tile(const GemmArgs& g, int& e, int& m_tile, int& n_tile) {
    const int r_pad = g.scalars[0];
    const int nt = g.N / kBN;
    const int total = (r_pad / BM) * nt;
    const int share = (total + kNumXcd - 1) / kNumXcd;
    const int xcd = blockIdx.x % kNumXcd, slot = blockIdx.x / kNumXcd;
    if (slot >= share) return false;
    const int L = xcd * share + slot;
    if (L >= total) return false;
    int lo = 0, hi = g.E - 1;  // largest e with first-tile(e) <= L
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((g.offsets[mid] / BM) * nt <= L) lo = mid; else hi = mid - 1;
    }
    e = lo;
    const int mb0 = g.offsets[e] / BM;
    const int mt = g.offsets[e + 1] / BM - mb0;
    const int local = L - mb0 * nt;
    n_tile = local / mt;
    m_tile = mb0 + local % mt;
    return true;
}

__device__ __forceinline__ float bf16_round(float v) { return (float)(__bf16)v; }

__device__ __forceinline__ uint16_t bf16_bits(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

// UE8M0 code of the smallest power of two 2^s with amax / 2^s <= 448, from
// the exponent and mantissa bits (448 = 1.75 * 2^8).
__device__ __forceinline__ int requant_code(float amax) {
    const uint32_t bits = __float_as_uint(amax);
    const int c = (int)(bits >> 23) - 8 + ((bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    return c < 0 ? 0 : c;
}

__device__ __forceinline__ float pow2_neg(int code) {  // 2^(127 - code), code in [0, 247]
    return __uint_as_float((uint32_t)(254 - code) << 23);
}

template <int BM, bool L1>
struct Smem {
    static constexpr int kA = BM * kBK;                     // one A stage
    static constexpr int kMain = 2 * kA + 2 * BM * 4;        // A stages + scale words
    static constexpr int kEpi = L1 ? BM * (kBN / 2) : BM * kBN * 2;
    static constexpr int kBytes = (kMain > kEpi ? kMain : kEpi);
};

template <int BM, bool L1>
__global__ __launch_bounds__(kThreads, BM >= 128 ? 1 : 2) void gemm_kernel(GemmArgs g) {
    constexpr int MI = BM / 16;
    constexpr int A_CHUNKS = BM * (kBK / 16);
    constexpr int A_PER = (A_CHUNKS + kThreads - 1) / kThreads;
    using S = Smem<BM, L1>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[S::kBytes];
    __shared__ float row_w[BM];
    __shared__ int row_tok[BM];

    int e, m_tile, n_tile;
    if (!map_tile<BM>(g, e, m_tile, n_tile)) return;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r0 = m_tile * BM;
    const int K = g.K, N = g.N;
    const int ksf = K / 32;          // scale bytes per row
    const int KT = K / kBK;

    if (tid < BM) {
        const int tok = g.row_token[r0 + tid];
        row_tok[tid] = tok;
        if (L1) row_w[tid] = tok >= 0 ? g.topk_w[(size_t)tok * g.topk + g.row_topk[r0 + tid]] : 0.0f;
    }
    __syncthreads();

    // ---- A-load assignment: chunk c -> (row c/8, 16-byte chunk c%8).  Offsets are
    // 32-bit (the host checks that every operand's row span stays below 2^31).
    constexpr uint32_t kNone = 0xFFFFFFFFu;
    uint32_t a_off[A_PER], a_sf_off[A_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
        const int c = tid + i * kThreads;
        a_off[i] = kNone;
        a_sf_off[i] = kNone;
        if (c < A_CHUNKS) {
            const int row = c >> 3;
            const int src_row = L1 ? row_tok[row] : r0 + row;
            if (src_row >= 0) {
                a_off[i] = (uint32_t)src_row * (uint32_t)K + (uint32_t)((c & 7) * 16);
                if ((c & 7) == 0) a_sf_off[i] = (uint32_t)src_row * (uint32_t)(ksf / 4);
            }
        }
    }
    const uint8_t* __restrict__ a_base = g.a;
    const uint32_t* __restrict__ a_sf_base = reinterpret_cast<const uint32_t*>(g.a_sf);
    v4i a_reg[A_PER];
    uint32_t s_reg[A_PER];
    auto load_a = [&](int kt) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            a_reg[i] = v4i{0, 0, 0, 0};
            s_reg[i] = 0x7F7F7F7Fu;
            if (a_off[i] != kNone) a_reg[i] = *reinterpret_cast<const v4i*>(a_base + a_off[i] + (uint32_t)kt * kBK);
            if (a_sf_off[i] != kNone) s_reg[i] = a_sf_base[a_sf_off[i] + kt];
        }
    };
    auto store_a = [&](int buf) {
        uint8_t* A = smem + buf * S::kA;
        uint32_t* SA = reinterpret_cast<uint32_t*>(smem + 2 * S::kA) + buf * BM;
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int c = tid + i * kThreads;
            if (c < A_CHUNKS) {
                const int row = c >> 3, ch = c & 7;
                *reinterpret_cast<v4i*>(A + row * kBK + ((ch ^ (row & 7)) << 4)) = a_reg[i];
                if (ch == 0) SA[row] = s_reg[i];
            }
        }
    };

    // ---- B: this lane's 4 columns (one per 16-column MFMA tile), from the expert's slab
    const int gq = lane >> 4;
    const uint8_t* __restrict__ b_base = g.b + (size_t)e * N * (K / 2);
    const uint32_t* __restrict__ b_sf_base = reinterpret_cast<const uint32_t*>(g.b_sf + (size_t)e * N * ksf);
    const uint32_t col0 = (uint32_t)(n_tile * kBN + w * 64 + (lane & 15));
    const uint32_t b_off0 = col0 * (uint32_t)(K / 2) + gq * 16;
    const uint32_t b_sf_off0 = col0 * (uint32_t)(ksf / 4);
    v4i b_cur[4], b_nxt[4];
    uint32_t bs_cur[4], bs_nxt[4];
    auto load_b = [&](int kt, v4i* bd, uint32_t* bs) {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            bd[ni] = *reinterpret_cast<const v4i*>(b_base + b_off0 + (uint32_t)(ni * 16 * (K / 2)) +
                                                   (uint32_t)kt * (kBK / 2));
            bs[ni] = b_sf_base[b_sf_off0 + (uint32_t)(ni * 16 * (ksf / 4)) + kt] >> (8 * gq);
        }
    };

    v4f acc[MI][4];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

    load_a(0);
    load_b(0, b_cur, bs_cur);
    store_a(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) {
            load_a(kt + 1);
            load_b(kt + 1, b_nxt, bs_nxt);
        }
        const uint8_t* A = smem + buf * S::kA;
        const uint32_t* SA = reinterpret_cast<const uint32_t*>(smem + 2 * S::kA) + buf * BM;
        v8i bfrag[4];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
            bfrag[ni] = v8i{b_cur[ni][0], b_cur[ni][1], b_cur[ni][2], b_cur[ni][3], 0, 0, 0, 0};
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int row = mi * 16 + (lane & 15);
            const v4i lo = *reinterpret_cast<const v4i*>(A + row * kBK + ((gq ^ (row & 7)) << 4));
            const v4i hi = *reinterpret_cast<const v4i*>(A + row * kBK + (((4 + gq) ^ (row & 7)) << 4));
            const v8i afrag = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const int sa = (int)(SA[row] >> (8 * gq));
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afrag, bfrag[ni], acc[mi][ni], 0, 4,
                                                                                0, sa, 0, (int)bs_cur[ni]);
        }
        if (kt + 1 < KT) {
            store_a(buf ^ 1);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                b_cur[ni] = b_nxt[ni];
                bs_cur[ni] = bs_nxt[ni];
            }
        }
        __syncthreads();
    }

    if constexpr (L1) {
        // ---- SwiGLU x w -> amax -> UE8M0 -> FP8, staged through LDS
        uint8_t* stage = smem;  // [BM][128] channel bytes of this tile
        const bool gate_lane = (lane & 8) == 0;
        const int ch_local = 32 * w + (lane & 7);
        const int n_sf = N / 64;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            v4f other[4];
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int c = 0; c < 4; ++c) other[ni][c] = __shfl_xor(acc[mi][ni][c], 8, 64);
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                const int i = gate_lane ? ii : 2 + ii;
                const int row_local = mi * 16 + 4 * (lane >> 4) + i;
                const float wgt = row_w[row_local];
                float h[4];
                float amax = 0.0f;
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) {
                    const float zg = gate_lane ? acc[mi][ni][i] : other[ni][i];
                    const float zu = gate_lane ? other[ni][i] : acc[mi][ni][i];
                    const float gv = bf16_round(zg);
                    const float uv = bf16_round(zu);
                    const float s = gv / (1.0f + expf(-gv));
                    h[ni] = (s * uv) * wgt;
                    amax = fmaxf(amax, fabsf(h[ni]));
                }
                amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
                amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
                amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
                const int code = requant_code(amax);
                const float inv = pow2_neg(code);
                const int q01 = __builtin_amdgcn_cvt_pk_fp8_f32(h[0] * inv, h[1] * inv, 0, false);
                const int q23 = __builtin_amdgcn_cvt_pk_fp8_f32(h[2] * inv, h[3] * inv, 0, false);
                uint8_t* srow = stage + row_local * (kBN / 2) + ch_local;
                srow[0] = (uint8_t)(q01 & 0xFF);
                srow[8] = (uint8_t)((q01 >> 8) & 0xFF);
                srow[16] = (uint8_t)(q23 & 0xFF);
                srow[24] = (uint8_t)((q23 >> 8) & 0xFF);
                if ((lane & 7) == 0) g.out_sf[(size_t)(r0 + row_local) * n_sf + n_tile * 4 + w] = (uint8_t)code;
            }
        }
        __syncthreads();
        const int n_q = N / 2;
        for (int c = tid; c < BM * 8; c += kThreads) {
            const int row = c >> 3, ch = c & 7;
            *reinterpret_cast<v4i*>(g.out_q + (size_t)(r0 + row) * n_q + n_tile * 128 + ch * 16) =
                *reinterpret_cast<const v4i*>(stage + row * 128 + ch * 16);
        }
    } else {
        // ---- FP32 -> BF16, staged through LDS, padding rows skipped
        uint16_t* stage = reinterpret_cast<uint16_t*>(smem);  // [BM][256]
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row_local = mi * 16 + 4 * (lane >> 4) + i;
                    const int col_local = w * 64 + ni * 16 + (lane & 15);
                    stage[row_local * kBN + col_local] = bf16_bits(acc[mi][ni][i]);
                }
        __syncthreads();
        for (int c = tid; c < BM * 32; c += kThreads) {
            const int row = c >> 5, ch = c & 31;
            if (row_tok[row] < 0) continue;
            *reinterpret_cast<v4i*>(g.out_bf16 + (size_t)(r0 + row) * N + n_tile * kBN + ch * 8) =
                *reinterpret_cast<const v4i*>(stage + row * kBN + ch * 8);
        }
    }
}

template <bool L1>
hipError_t launch_gemm(const GemmProblem& p, const GemmArgs& args, hipStream_t stream) {
    const int bm = p.shape->block_m;
    const int64_t tiles = (p.cap / bm) * (args.N / kBN);
    const int64_t grid = (tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (grid == 0) return hipSuccess;
    switch (bm) {
        case 16: hipLaunchKernelGGL((gemm_kernel<16, L1>), dim3(grid), dim3(kThreads), 0, stream, args); break;
        case 32: hipLaunchKernelGGL((gemm_kernel<32, L1>), dim3(grid), dim3(kThreads), 0, stream, args); break;
        case 64: hipLaunchKernelGGL((gemm_kernel<64, L1>), dim3(grid), dim3(kThreads), 0, stream, args); break;
        case 128: hipLaunchKernelGGL((gemm_kernel<128, L1>), dim3(grid), dim3(kThreads), 0, stream, args); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_linear1(const GemmProblem& p, const uint8_t* x, const uint8_t* x_sf, const float* topk_w,
                          const uint8_t* w1, const uint8_t* w1_sf, uint8_t* h_q, uint8_t* h_sf,
                          hipStream_t stream) {
    GemmArgs a{};
    a.a = x; a.a_sf = x_sf; a.b = w1; a.b_sf = w1_sf;
    a.scalars = p.plan->scalars; a.offsets = p.plan->offsets;
    a.row_token = p.plan->row_token; a.row_topk = p.plan->row_topk;
    a.topk_w = topk_w; a.out_q = h_q; a.out_sf = h_sf; a.out_bf16 = nullptr;
    a.K = p.shape->hidden; a.N = 2 * p.shape->intermediate; a.E = p.shape->num_experts; a.topk = p.shape->topk;
    return launch_gemm<true>(p, a, stream);
}

hipError_t launch_linear2(const GemmProblem& p, const uint8_t* h_q, const uint8_t* h_sf, const uint8_t* w2,
                          const uint8_t* w2_sf, uint16_t* yslot, hipStream_t stream) {
    GemmArgs a{};
    a.a = h_q; a.a_sf = h_sf; a.b = w2; a.b_sf = w2_sf;
    a.scalars = p.plan->scalars; a.offsets = p.plan->offsets;
    a.row_token = p.plan->row_token; a.row_topk = p.plan->row_topk;
    a.topk_w = nullptr; a.out_q = nullptr; a.out_sf = nullptr; a.out_bf16 = yslot;
    a.K = p.shape->intermediate; a.N = p.shape->hidden; a.E = p.shape->num_experts; a.topk = p.shape->topk;
    return launch_gemm<false>(p, a, stream);
}

}  // namespace moe
