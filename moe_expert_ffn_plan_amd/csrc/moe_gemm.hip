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
//  * Workgroup tile BM x BN (BN = 512 with 8 waves when N allows, else 256
//    with 4 waves), waves in a WM x WN grid.  A wave's columns are a
//    multiple of 64 (= 32 gate/up channels = one requant scale group), so the
//    amax reduction stays inside a wave.
//  * Operands stream through a ring of NS LDS stages, each one 128-wide
//    K-step of A (BM x 128 B), B (BN x 64 B) and both scale words, filled by
//    global_load_lds DMA so in-flight tiles cost no registers.  Each wave
//    issues exactly D_W DMA instructions per stage (every lane active, every
//    address valid), so "stage kt has landed" is s_waitcnt vmcnt(n * D_W)
//    with n the stages issued after it, followed by a workgroup barrier.  The
//    DMA is issued from inline asm so the compiler does not add its own
//    whole-queue waits in front of every LDS read.
//  * Weights and their scales come pre-tiled (moe_prepare.hip): a stage's B
//    is one contiguous block already in LDS order, so every DMA instruction
//    moves 1 KiB of contiguous memory.  A chunks are XOR-swizzled in LDS
//    (chunk ^ ((row >> 1) & 7)), B chunks by the tiling (chunk ^ ((col >> 2)
//    & 3)), so the MFMA-pattern ds_read_b128s of 16 consecutive rows/columns
//    hit distinct banks.
//  * Tiles come from a list (expert by expert; for each N-tile all M-tiles
//    of the expert) and blockIdx is remapped so that each XCD (blockIdx % 8
//    on MI300-class parts) runs a contiguous run of that list: the M-tiles
//    sharing a weight tile run together on one XCD and hit its L2.
#include "moe_internal.h"

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBK = 128;
constexpr int kTileN = 256;  // width of one tiled-weight block (moe_prepare.hip)
constexpr int kNumXcd = 8;

struct GemmArgs {
    const uint8_t* a;      // Linear1: x [T, K]; Linear2: h_q [cap, K]
    const uint8_t* a_sf;   // per-row-block scales [cap/BM][K/128][BM][4]
    const uint8_t* b;      // tiled weights [E][N/256][K/128][1024 x 16 B]
    const uint8_t* b_sf;   // tiled weight scales [E][N/256][K/128][256][4]
    const int32_t* scalars;
    const int32_t* tiles;  // {m_tile, n_tile << 16 | e} per tile
    const int32_t* row_token;
    const float* row_w;    // Linear1: per-row top-k weight
    uint8_t* out_q;        // Linear1: [cap, N/2]
    uint8_t* out_sf;       // Linear1: per-row-block scales [cap/BM][N/256][BM][4]
    uint16_t* out_bf16;    // Linear2: [cap, N]
    int K, N;
};

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

// ---- LDS DMA: lane l writes `size` bytes at LDS address m0 + l * size.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
    asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}
// Wait until at most N DMA instructions of this wave are in flight and this
// wave's LDS reads are done, then meet the other waves.
template <int N>
__device__ __forceinline__ void wait_stage_and_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

template <int BM, int BN, int NW>
struct Cfg {
    static constexpr int THREADS = 64 * NW;
    static constexpr int WM = BM >= 128 ? 2 : 1;       // wave grid rows
    static constexpr int WN = NW / WM;                  // wave grid cols
    static constexpr int WTM = BM / WM;                 // wave tile rows
    static constexpr int WTN = BN / WN;                 // wave tile cols
    static_assert(WTN % 64 == 0, "a wave must own whole 64-column requant groups");
    static constexpr int MI = WTM / 16;
    static constexpr int NI = WTN / 16;
    static constexpr int A_BYTES = BM * kBK;
    static constexpr int B_BYTES = BN * (kBK / 2);
    static constexpr int SA_WORDS = BM > 64 ? BM : 64;  // one DMA instruction covers 64 rows
    static constexpr int SB_WORDS = BN;
    static constexpr int STAGE = A_BYTES + B_BYTES + 4 * SA_WORDS + 4 * SB_WORDS;
    static constexpr int NS = (152 * 1024) / STAGE >= 4 ? 4 : 3;  // LDS stages
    static constexpr int A_INSTR = A_BYTES / 1024;      // 1 KiB per wave DMA instruction
    static constexpr int A_PW = A_INSTR >= NW ? A_INSTR / NW : 1;
    static constexpr int B_PW = B_BYTES / 1024 / NW;
    static constexpr int SA_INSTR = SA_WORDS / 64;
    static constexpr int SB_INSTR = SB_WORDS / 64;
    static constexpr int SB_PW = SB_INSTR >= NW ? SB_INSTR / NW : 1;
    static constexpr int D_W = A_PW + B_PW + 1 + SB_PW;  // DMA instructions per wave per stage
    static_assert(A_INSTR % NW == 0 || A_INSTR < NW, "A instructions must split evenly");
    static_assert((B_BYTES / 1024) % NW == 0, "B instructions must split evenly");
    static_assert(2 * D_W < 64, "vmcnt range");
};

template <int BM, int BN, int NW, bool L1>
struct Smem {
    using C = Cfg<BM, BN, NW>;
    static constexpr int kMain = C::NS * C::STAGE;
    static constexpr int kEpi = L1 ? BM * (BN / 2) : BM * BN * 2;
    static constexpr int kBytes = (kMain > kEpi ? kMain : kEpi);
};

template <int BM, int BN, int NW, bool L1>
__global__ __launch_bounds__(64 * NW, 1) void gemm_kernel(GemmArgs g) {
    using C = Cfg<BM, BN, NW>;
    using S = Smem<BM, BN, NW, L1>;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[S::kBytes];
    __shared__ float row_w[BM];
    __shared__ int row_tok[BM];

    // ---- tile of this workgroup (XCD-contiguous runs of the tile list)
    const int nt = g.N / BN;
    const int total = (g.scalars[0] / BM) * nt;
    const int share = (total + kNumXcd - 1) / kNumXcd;
    const int slot = blockIdx.x / kNumXcd;
    if (slot >= share) return;
    const int L = (blockIdx.x % kNumXcd) * share + slot;
    if (L >= total) return;
    const int m_tile = g.tiles[2 * L];
    const int n_tile = g.tiles[2 * L + 1] >> 16;
    const int e = g.tiles[2 * L + 1] & 0xFFFF;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r0 = m_tile * BM;
    const int K = g.K, N = g.N;
    const int KT = K / kBK;

    if (tid < BM) {
        row_tok[tid] = g.row_token[r0 + tid];
        if (L1) row_w[tid] = g.row_w[r0 + tid];
    }
    __syncthreads();

    // ---- per-lane DMA sources
    uint32_t a_off[C::A_PW];
#pragma unroll
    for (int i = 0; i < C::A_PW; ++i) {
        const int blk = (i * NW + w) % C::A_INSTR;
        const int p = blk * 64 + lane;             // 16-byte LDS slot of this lane
        const int row = p >> 3;
        const int c = (p & 7) ^ ((row >> 1) & 7);  // logical chunk stored in that slot
        int src_row;
        if (L1) {
            const int t = row_tok[row];
            src_row = t >= 0 ? t : 0;              // padding rows read token 0 (their weight is 0)
        } else {
            src_row = r0 + row;
        }
        a_off[i] = (uint32_t)src_row * (uint32_t)K + (uint32_t)(c * 16);
    }
    // tiled weights: stage kt of one 256-column block is 16 KiB (+1 KiB of scales), contiguous
    const int tn0 = n_tile * (BN / kTileN);  // first 256-column block of this tile
    const size_t tb0 = ((size_t)e * (N / kTileN) + tn0) * KT;
    const uint8_t* a_base = g.a;
    const int sa_blk = w % C::SA_INSTR;
    const uint8_t* a_sf_base = g.a_sf + (size_t)m_tile * KT * (4 * BM) + min(sa_blk * 64 + lane, BM - 1) * 4;

    auto issue_stage = [&](int kt) {
        uint8_t* st = smem + (kt % C::NS) * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::A_PW; ++i) {
            const int blk = (i * NW + w) % C::A_INSTR;
            dma16(a_base + a_off[i] + (uint32_t)kt * kBK, lds_addr(st + blk * 1024));
        }
#pragma unroll
        for (int i = 0; i < C::B_PW; ++i) {
            const int blk = i * NW + w;          // 1 KiB block of this stage's B (16 per 256 columns)
            const uint8_t* src = g.b + ((tb0 + (size_t)(blk >> 4) * KT + kt) * 16 + (blk & 15)) * 1024 + lane * 16;
            dma16(src, lds_addr(st + C::A_BYTES + blk * 1024));
        }
        dma4(a_sf_base + (size_t)kt * (4 * BM), lds_addr(st + C::A_BYTES + C::B_BYTES + sa_blk * 256));
#pragma unroll
        for (int i = 0; i < C::SB_PW; ++i) {
            const int blk = (i * NW + w) % C::SB_INSTR;  // 64 columns per instruction
            const uint8_t* src = g.b_sf + ((tb0 + (size_t)(blk >> 2) * KT + kt) * 256 + (blk & 3) * 64 + lane) * 4;
            dma4(src, lds_addr(st + C::A_BYTES + C::B_BYTES + 4 * C::SA_WORDS + blk * 256));
        }
    };

    const int wm = w / C::WN, wn = w % C::WN;
    const int gq = lane >> 4;
    v4f acc[C::MI][C::NI];
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int s = 0; s < C::NS - 1; ++s)
        if (s < KT) issue_stage(s);

    for (int kt = 0; kt < KT; ++kt) {
        const int after = min(C::NS - 2, KT - 1 - kt);  // stages issued after kt
        if (after >= 2) wait_stage_and_barrier<2 * C::D_W>();
        else if (after == 1) wait_stage_and_barrier<C::D_W>();
        else wait_stage_and_barrier<0>();
        if (kt + C::NS - 1 < KT) issue_stage(kt + C::NS - 1);

        const uint8_t* st = smem + (kt % C::NS) * C::STAGE;
        const uint8_t* A = st;
        const uint8_t* Bt = st + C::A_BYTES;
        const uint32_t* SA = reinterpret_cast<const uint32_t*>(st + C::A_BYTES + C::B_BYTES);
        const uint32_t* SB = SA + C::SA_WORDS;
        v8i bfrag[C::NI];
        int sb[C::NI];
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni) {
            const int col = wn * C::WTN + ni * 16 + (lane & 15);
            const v4i b = *reinterpret_cast<const v4i*>(Bt + col * (kBK / 2) + ((gq ^ ((col >> 2) & 3)) << 4));
            bfrag[ni] = v8i{b[0], b[1], b[2], b[3], 0, 0, 0, 0};
            sb[ni] = (int)(SB[col] >> (8 * gq));
        }
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi) {
            const int row = wm * C::WTM + mi * 16 + (lane & 15);
            const int sw = (row >> 1) & 7;
            const v4i lo = *reinterpret_cast<const v4i*>(A + row * kBK + ((gq ^ sw) << 4));
            const v4i hi = *reinterpret_cast<const v4i*>(A + row * kBK + (((4 + gq) ^ sw) << 4));
            const v8i afrag = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const int sa = (int)(SA[row] >> (8 * gq));
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afrag, bfrag[ni], acc[mi][ni], 0, 4,
                                                                                0, sa, 0, sb[ni]);
        }
    }
    __syncthreads();  // every wave is done with the stages before they are reused below

    if constexpr (L1) {
        // ---- SwiGLU x w -> amax -> UE8M0 -> FP8, staged through LDS
        uint8_t* stage = smem;  // [BM][BN/2] channel bytes of this tile
        const bool gate_lane = (lane & 8) == 0;
        const int ksteps2 = N / kTileN;  // Linear2 K-steps (128 channels each)
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi) {
            v4f other[C::NI];
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
                for (int c = 0; c < 4; ++c) other[ni][c] = __shfl_xor(acc[mi][ni][c], 8, 64);
#pragma unroll
            for (int grp = 0; grp < C::NI / 4; ++grp) {  // 64 columns = 32 channels = one scale group
                const int col0 = wn * C::WTN + grp * 64;  // first column of the group in this tile
                const int ch0 = col0 / 2 + (lane & 7);
#pragma unroll
                for (int ii = 0; ii < 2; ++ii) {
                    const int i = gate_lane ? ii : 2 + ii;
                    const int row_local = wm * C::WTM + mi * 16 + 4 * (lane >> 4) + i;
                    const float wgt = row_w[row_local];
                    float h[4];
                    float amax = 0.0f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int ni = grp * 4 + q;
                        const float zg = gate_lane ? acc[mi][ni][i] : other[ni][i];
                        const float zu = gate_lane ? other[ni][i] : acc[mi][ni][i];
                        const float gv = bf16_round(zg);
                        const float uv = bf16_round(zu);
                        const float s = gv / (1.0f + expf(-gv));
                        h[q] = (s * uv) * wgt;
                        amax = fmaxf(amax, fabsf(h[q]));
                    }
                    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
                    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
                    amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
                    const int code = requant_code(amax);
                    const float inv = pow2_neg(code);
                    const int q01 = __builtin_amdgcn_cvt_pk_fp8_f32(h[0] * inv, h[1] * inv, 0, false);
                    const int q23 = __builtin_amdgcn_cvt_pk_fp8_f32(h[2] * inv, h[3] * inv, 0, false);
                    uint8_t* srow = stage + row_local * (BN / 2) + ch0;
                    srow[0] = (uint8_t)(q01 & 0xFF);
                    srow[8] = (uint8_t)((q01 >> 8) & 0xFF);
                    srow[16] = (uint8_t)(q23 & 0xFF);
                    srow[24] = (uint8_t)((q23 >> 8) & 0xFF);
                    // Linear2 K-step = 256-column block of this tile's Z, byte = group within it
                    if ((lane & 7) == 0) {
                        const int gcol = n_tile * BN + col0;
                        g.out_sf[(((size_t)m_tile * ksteps2 + gcol / kTileN) * BM + row_local) * 4 +
                                 (gcol % kTileN) / 64] = (uint8_t)code;
                    }
                }
            }
        }
        __syncthreads();
        const int n_q = N / 2;
        constexpr int CPR = BN / 32;  // 16-byte chunks per staged row
        for (int c = tid; c < BM * CPR; c += C::THREADS) {
            const int row = c / CPR, ch = c % CPR;
            *reinterpret_cast<v4i*>(g.out_q + (size_t)(r0 + row) * n_q + n_tile * (BN / 2) + ch * 16) =
                *reinterpret_cast<const v4i*>(stage + row * (BN / 2) + ch * 16);
        }
    } else {
        // ---- FP32 -> BF16, staged through LDS, padding rows skipped
        uint16_t* stage = reinterpret_cast<uint16_t*>(smem);  // [BM][BN]
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row_local = wm * C::WTM + mi * 16 + 4 * (lane >> 4) + i;
                    const int col_local = wn * C::WTN + ni * 16 + (lane & 15);
                    stage[row_local * BN + col_local] = bf16_bits(acc[mi][ni][i]);
                }
        __syncthreads();
        constexpr int CPR = BN / 8;
        for (int c = tid; c < BM * CPR; c += C::THREADS) {
            const int row = c / CPR, ch = c % CPR;
            if (row_tok[row] < 0) continue;
            *reinterpret_cast<v4i*>(g.out_bf16 + (size_t)(r0 + row) * N + n_tile * BN + ch * 8) =
                *reinterpret_cast<const v4i*>(stage + row * BN + ch * 8);
        }
    }
}

template <int BM, bool L1>
hipError_t launch_bm(const GemmArgs& args, int64_t grid, hipStream_t stream) {
    if (gemm_bn(args.N) == 512)
        hipLaunchKernelGGL((gemm_kernel<BM, 512, 8, L1>), dim3(grid), dim3(512), 0, stream, args);
    else
        hipLaunchKernelGGL((gemm_kernel<BM, 256, 4, L1>), dim3(grid), dim3(256), 0, stream, args);
    return hipGetLastError();
}

template <bool L1>
hipError_t launch_gemm(const GemmProblem& p, const GemmArgs& args, hipStream_t stream) {
    const int bm = p.shape->block_m;
    const int64_t tiles = (p.cap / bm) * (args.N / gemm_bn(args.N));
    const int64_t grid = (tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (grid == 0) return hipSuccess;
    switch (bm) {
        case 16: return launch_bm<16, L1>(args, grid, stream);
        case 32: return launch_bm<32, L1>(args, grid, stream);
        case 64: return launch_bm<64, L1>(args, grid, stream);
        case 128: return launch_bm<128, L1>(args, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

GemmArgs common_args(const GemmProblem& p) {
    GemmArgs a{};
    a.scalars = p.plan->scalars;
    a.tiles = p.tiles;
    a.row_token = p.plan->row_token;
    a.row_w = p.row_w;
    return a;
}

}  // namespace

hipError_t launch_linear1(const GemmProblem& p, const uint8_t* x, const uint8_t* x_sf_tiled, const uint8_t* w1,
                          const uint8_t* w1_sf, uint8_t* h_q, uint8_t* h_sf, hipStream_t stream) {
    GemmArgs a = common_args(p);
    a.a = x; a.a_sf = x_sf_tiled; a.b = w1; a.b_sf = w1_sf;
    a.out_q = h_q; a.out_sf = h_sf; a.out_bf16 = nullptr;
    a.K = p.shape->hidden; a.N = 2 * p.shape->intermediate;
    return launch_gemm<true>(p, a, stream);
}

hipError_t launch_linear2(const GemmProblem& p, const uint8_t* h_q, const uint8_t* h_sf, const uint8_t* w2,
                          const uint8_t* w2_sf, uint16_t* yslot, hipStream_t stream) {
    GemmArgs a = common_args(p);
    a.a = h_q; a.a_sf = h_sf; a.b = w2; a.b_sf = w2_sf;
    a.out_q = nullptr; a.out_sf = nullptr; a.out_bf16 = yslot;
    a.K = p.shape->intermediate; a.N = p.shape->hidden;
    return launch_gemm<false>(p, a, stream);
}

}  // namespace moe
