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
//  * Operands stream through a ring of NS LDS stages, each one 128-wide
//    K-step of A (BM x 128 B), B (BN x 64 B) and both scale words, filled by
//    global_load_lds DMA so in-flight tiles cost no registers.  Every wave
//    issues a fixed number of DMA instructions per stage (every lane active,
//    every address valid), so "this wave's share of stage s has landed" is
//    s_waitcnt vmcnt(n * D) with n the stages it issued after s; a workgroup
//    barrier after that wait makes the whole stage visible.  The DMA is
//    issued from inline asm so the compiler does not add its own whole-queue
//    waits in front of every LDS read.
//  * Weights and their scales come pre-tiled (moe_prepare.hip): a stage's B
//    is one contiguous block already in LDS order, so every DMA instruction
//    moves 1 KiB of contiguous memory, and the columns are permuted so that
//    each lane's outputs are adjacent in memory: four channels of a 64-column
//    group in Linear1 (one FP8 dword), eight columns of a 128-column span in
//    Linear2 (a 16-byte BF16 run; 8 bytes for 64-column wave tiles), stored
//    straight from the accumulators.  A chunks are XOR-swizzled in LDS (chunk ^ ((row >> 1)
//    & 7)), B chunks by the tiling (chunk ^ ((col >> 1) & 3)).  Measured on
//    the device, a ds_read_b128 runs without bank conflicts when the lanes
//    l, l^2, l^4, l^6 of each group address distinct 16-byte slots modulo
//    128 bytes; both swizzles give that for the MFMA fragment reads of 16
//    consecutive rows or columns (with chunk ^ ((col >> 2) & 3) the B reads
//    were two-way conflicted).
//  * 512-column tiles run 8 waves as two groups of four that alternate
//    ("ping-pong"): while one group issues the MFMAs of its K-step, the other
//    issues its share of the DMA and reads its next fragments from LDS, with
//    one workgroup barrier per K-step.  The two waves sharing a SIMD are
//    thus rarely both away from the matrix core, which a single group of
//    barrier-synchronised waves cannot avoid.  Group 0 streams most of the
//    weights, group 1 the activation rows and the rest of the weights.
//    256-column tiles (small N) use one group of four waves that reads, then
//    multiplies.
//  * Tiles come from a list (expert by expert, M-tile by M-tile, all N-tiles
//    of each).  An M-tile spans up to 128 rows, several routing blocks of one
//    expert, so a weight tile is fetched once per 128 rows rather than once
//    per block; rows past the expert's last hit are masked.  blockIdx is remapped
//    so that each XCD (blockIdx % 8) runs a contiguous range of M-tiles: the
//    M-tiles sharing a weight tile run together on one XCD and hit its L2.
#include "moe_internal.h"

#include <algorithm>
#include <atomic>

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBK = 128;
constexpr int kTileN = 256;  // width of one tiled-weight block (moe_prepare.hip)
constexpr int kNumXcd = 8;
constexpr int kLdsBudget = 155 * 1024;  // operand ring; the rest of the 160 KiB holds per-row tables

struct GemmArgs {
    const uint8_t* a;       // Linear1: x [T, K]; Linear2: h_q [cap, K]
    const uint8_t* a_sf;    // Linear1: x_sf [T, K/32]; Linear2: per-block scales [cap/bm][K/128][bm][4]
    const uint8_t* b;       // tiled weights [E][N/256][K/128][1024 x 16 B]
    const uint8_t* b_sf;    // tiled weight scales [E][N/256][K/128][256][4]
    const int32_t* scalars;
    const int32_t* tiles;   // {first row, n_tile << 16 | e, valid rows, M-tile index} per tile
    const int32_t* row_token;
    const int32_t* row_topk;
    const float* topk_w;    // Linear1: top-k weights [T, k]
    uint8_t* out_q;         // Linear1: [cap, N/2]
    uint8_t* out_sf;        // Linear1: per-block scales [cap/bm][N/256][bm][4]
    uint16_t* out_bf16;     // Linear2: [cap, N]
    int K, N, topk;
    int bm;                 // the routing block (block_m) that the scale layout uses
    int bm_shift;           // log2(bm) when bm is a power of two, else -1
    float swiglu_limit;     // Linear1: > 0 clamps gate from above and up on both sides before SwiGLU
    int exact_silu;         // Linear1: 1 = accurate expf and IEEE division in SiLU
    int count_idx;          // scalars[count_idx] = tiles in the list
    uint32_t* status;       // Linear1 launched on its own: the forward's status word, cleared by workgroup 0
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to BF16 (round to nearest even) with one v_cvt_pk_bf16_f32: lo in bits 0-15.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

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

// Cross-lane moves inside a 16-lane row (DPP, no LDS round trip).  Every control used here stays
// inside the row, so no lane reads out of range.
constexpr int kDppXor1 = 0xB1;         // lane i <- lane i ^ 1 (quad_perm [1, 0, 3, 2])
constexpr int kDppXor2 = 0x4E;         // lane i <- lane i ^ 2 (quad_perm [2, 3, 0, 1])
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane i ^ 7 (mirror within each group of 8)
constexpr int kDppRowMirror = 0x140;   // lane i <- lane i ^ 15 (mirror within the row)

// Maxima of non-negative floats are taken on their bit patterns, which order the same way; the
// integer maximum also needs no NaN quieting of the moved operand, so it fuses with the DPP move.
template <int CTRL>
__device__ __forceinline__ uint32_t umax_dpp(uint32_t a, uint32_t b) {
    return max(a, (uint32_t)__builtin_amdgcn_mov_dpp((int)b, CTRL, 0xF, 0xF, true));
}
// One step of a transposed maximum: the lane and its partner (which differs from it in the step's
// split bit) each keep one half of their first N values and take the partner's copy of that half.
template <int CTRL, int N, int V>
__device__ __forceinline__ void fold_half(uint32_t (&m)[V], bool upper) {
#pragma unroll
    for (int t = 0; t < N / 2; ++t) {
        const uint32_t keep = upper ? m[t + N / 2] : m[t];
        const uint32_t send = upper ? m[t] : m[t + N / 2];
        m[t] = umax_dpp<CTRL>(keep, send);
    }
}
// Maxima over the 16 lanes of each DPP row of V = 4 or 8 non-negative values per lane (as bit
// patterns): lane j returns the maximum of value j >> (V == 8 ? 1 : 2).  The partners of the four
// steps (j ^ 15, j ^ 7, j ^ 2, j ^ 1) span all 16 lanes; the first log2(V) steps split on bits 3, 2
// (and 1) of j, so each halving keeps the values whose index matches those bits.
template <int V>
__device__ __forceinline__ float row_max16(uint32_t (&m)[V], int j) {
    static_assert(V == 4 || V == 8, "four or eight values per lane");
    fold_half<kDppRowMirror, V>(m, j & 8);
    fold_half<kDppHalfMirror, V / 2>(m, j & 4);
    if constexpr (V == 8) fold_half<kDppXor2, 2>(m, j & 2);
    else m[0] = umax_dpp<kDppXor2>(m[0], m[0]);
    return __uint_as_float(umax_dpp<kDppXor1>(m[0], m[0]));
}

// ---- LDS DMA: lane l reads `size` bytes at the wave-uniform base plus its
// own 32-bit offset and writes them at LDS address m0 + l * size.
// The base must be wave-uniform; the compiler cannot always prove that of a
// pointer picked at run time from one of two argument blocks, so it is read
// from the first lane (free where it already sits in SGPRs).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}
// Lane index computed where it is used.  Code that runs once per tile takes
// it from here so the compiler recomputes the per-lane values it derives
// (two instructions) instead of keeping them live across the K-loop, where
// the registers are needed for fragments and accumulators.
__device__ __forceinline__ int fresh_lane() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
// The same with the non-temporal hint: for operands streamed about once (weight tiles of batches with
// few rows per expert), so they do not displace reused data in the caches.
__device__ __forceinline__ void dma16_stream(uint32_t voff, const void* sbase, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4(uint32_t voff, const void* sbase, uint32_t lds) {
    asm volatile("global_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
// Wait until at most N DMA instructions of this wave are in flight and this
// wave's LDS reads are done, then meet the other waves.  The scheduling
// barriers keep the compiler from moving MFMAs or LDS reads across it.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
    __builtin_amdgcn_sched_barrier(0);
}
// up to n (0..2) later stages of D instructions each, plus `extra` (0 or 1)
// further instructions issued with them, may stay in flight
template <int D>
__device__ __forceinline__ void wait_stages_and_barrier(int n, int extra = 0) {
    if (n >= 2) {
        if (extra) wait_and_barrier<2 * D + 1>();
        else wait_and_barrier<2 * D>();
    } else if (n == 1) {
        if (extra) wait_and_barrier<D + 1>();
        else wait_and_barrier<D>();
    } else {
        wait_and_barrier<0>();
    }
}
constexpr int kNoVmWait = 63;  // vmcnt field maximum: wait for LDS reads only

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// A tile: rows [m, m + BM) of expert e's rows, of which the first `rows` are
// the expert's (the rest belong to the next expert or lie past the table and
// are neither read through nor written), columns [n * BN, n * BN + BN).
struct TileId {
    int m, n, e, rows, mt;  // mt: M-tile index over all experts
};
// XCD xcd's part of a tile list with nt tiles per M-tile (the list runs
// M-tile by M-tile): the tiles of M-tiles [xcd * s, (xcd + 1) * s), s =
// ceil(M-tiles / 8), as list range [begin, end).  Both GEMMs' lists split
// into the same M-tiles, so an XCD's Linear2 tiles need only the rows its own
// Linear1 tiles computed, and the tiles sharing a weight tile (the M-tiles of
// one expert) run together on one XCD and hit its L2.
__device__ __forceinline__ void xcd_chunk(const GemmArgs& g, int nt, int xcd, int& begin, int& end) {
    const int mts = g.scalars[g.count_idx] / nt;
    const int share = (mts + kNumXcd - 1) / kNumXcd;
    begin = min(xcd * share, mts) * nt;
    end = min((xcd + 1) * share, mts) * nt;
}

// Tile of this workgroup (one tile per workgroup, blockIdx % 8 = XCD).
// False for the padding workgroups of the grid.
__device__ __forceinline__ bool tile_of_block(const GemmArgs& g, int BN, TileId& t) {
    int begin, end;
    xcd_chunk(g, g.N / BN, blockIdx.x % kNumXcd, begin, end);
    const int L = begin + blockIdx.x / kNumXcd;
    if (L >= end) return false;
    const int32_t* e = g.tiles + kTileWords * L;
    t.m = e[0];
    t.n = e[1] >> 16;
    t.e = e[1] & 0xFFFF;
    t.rows = e[2];
    t.mt = e[3];
    return true;
}

// Byte offset of row r's scale word of K-step 0 in the per-block layout
// [cap/bm][KT][bm][4]; K-step kt adds kt * bm * 4.  bm_shift = log2(bm) for a power of two, else -1
// (blocks of 96 and 192 rows divide).
__device__ __forceinline__ uint32_t block_scale_offset(int r, int KT, int bm, int bm_shift) {
    const int blk = bm_shift >= 0 ? r >> bm_shift : r / bm;
    return (uint32_t)((blk * KT) * bm + (r - blk * bm)) * 4u;
}
// The same for K-step kt of row m0 + row_local, m0 the first row of a tile:
// without PARTIAL the tile is one block of BM rows and m0 a multiple of BM.
template <int BM, bool PARTIAL>
__device__ __forceinline__ uint32_t tile_scale_offset(int m0, int row_local, int KT, int kt, int bm, int bm_shift) {
    if constexpr (PARTIAL)
        return block_scale_offset(m0 + row_local, KT, bm, bm_shift) + (uint32_t)(kt * bm) * 4u;
    else
        return (((uint32_t)m0 / BM * (uint32_t)KT + (uint32_t)kt) * BM + (uint32_t)row_local) * 4u;
}

// ---- operand layout of one LDS stage
template <int BM, int BN>
struct StageLayout {
    static constexpr int A_BYTES = BM * kBK;
    static constexpr int B_BYTES = BN * (kBK / 2);
    static constexpr int SA_WORDS = BM > 64 ? BM : 64;  // one DMA instruction covers 64 rows
    static constexpr int SB_WORDS = BN;
    static constexpr int STAGE = A_BYTES + B_BYTES + 4 * SA_WORDS + 4 * SB_WORDS;
    static constexpr int NS = kLdsBudget / STAGE >= 4 ? 4 : 3;
    static_assert(kLdsBudget / STAGE >= 3, "three stages must fit");
    static constexpr int A_INSTR = A_BYTES / 1024;  // 1 KiB per DMA instruction
    static constexpr int B_INSTR = B_BYTES / 1024;
    static constexpr int SA_INSTR = SA_WORDS / 64;   // gathered 4-byte words: 64 rows per instruction
    static constexpr int SB_INSTR = SB_WORDS / 256;  // contiguous: 256 columns (1 KiB) per instruction
    static_assert(SA_INSTR + SB_INSTR <= 4, "one scale instruction per A-side wave");
};

// DMA sources of one wave (STREAM: weight tiles loaded with the non-temporal hint, see issue_b_blocks).
// The A side (rows, and all scales) is split over `anw` waves, the weight blocks over `bnw` waves; where
// an operand has fewer instructions than waves, waves repeat one, writing the same bytes to the same
// place.  Each A-side wave issues one scale instruction per stage: waves 0 .. SA_INSTR-1 an activation-
// scale block, the next SB_INSTR waves a weight-scale block, any further wave a repeat of an
// activation-scale block.  Bases are wave-uniform (SGPRs); only the per-lane offsets live in VGPRs.
template <int BM, int BN, int A_PW, int B_PW, bool STREAM>
struct StageDma {
    using L = StageLayout<BM, BN>;
    uint32_t a_off[A_PW];  // gathered row * K + chunk
    uint32_t sa_off;       // Linear1: gathered row * K/32; Linear2: row * 4 in the row block
    const uint8_t* a;
    const uint8_t* a_sf;
    const uint8_t* b;
    const uint8_t* b_sf;
    int KT, aw, anw, bw, bnw, sa_blk, sa_kt, sb_blk;
    bool sb_wave;  // this wave's scale instruction loads weight scales

    // Linear1 gathers rows and their scales through row_token; its padding
    // rows read token 0 (their top-k weight is 0, so they produce h = 0).
    // Rows past the tile's valid count read token 0 (Linear1) or the tile's
    // first row (Linear2): their results are never stored.
    __device__ __forceinline__ void init_a(const GemmArgs& g, int m0, int rows, const int* row_tok, bool l1, int aw_,
                                           int anw_) {
        const int lane = fresh_lane();
        aw = aw_; anw = anw_;
        KT = g.K / kBK;
#pragma unroll
        for (int i = 0; i < A_PW; ++i) {
            const int blk = (i * anw + aw) % L::A_INSTR;
            const int p = blk * 64 + lane;             // 16-byte LDS slot of this lane
            const int row = p >> 3;
            const int c = (p & 7) ^ ((row >> 1) & 7);  // logical chunk stored in that slot
            int src_row;
            if (l1) {
                const int t = row < rows ? row_tok[row] : -1;
                src_row = t >= 0 ? t : 0;
            } else {
                src_row = m0 + (row < rows ? row : 0);
            }
            a_off[i] = (uint32_t)src_row * (uint32_t)g.K + (uint32_t)(c * 16);
        }
        a = static_cast<const uint8_t*>(uniform_ptr(g.a));
        sb_wave = aw >= L::SA_INSTR && aw < L::SA_INSTR + L::SB_INSTR;
        sb_blk = aw - L::SA_INSTR;
        sa_blk = aw % L::SA_INSTR;
        const int sa_row = min(sa_blk * 64 + lane, BM - 1);
        a_sf = static_cast<const uint8_t*>(uniform_ptr(g.a_sf));
        if (l1) {  // x_sf [T, K/32]: the 4 bytes of K-step kt of token t sit at t * K/32 + 4 kt
            const int t = sa_row < rows ? row_tok[sa_row] : -1;
            sa_off = (uint32_t)(t >= 0 ? t : 0) * (uint32_t)(g.K / 32);
            sa_kt = 4;
        } else {   // per-block layout [cap/bm][KT][bm][4]
            sa_off = block_scale_offset(m0 + (sa_row < rows ? sa_row : 0), KT, g.bm, g.bm_shift);
            sa_kt = 4 * g.bm;
        }
    }
    __device__ __forceinline__ void init_b(const GemmArgs& g, const TileId& t, int bw_, int bnw_) {
        bw = bw_; bnw = bnw_;
        KT = g.K / kBK;
        const int tn0 = t.n * (BN / kTileN);  // first 256-column block of this tile
        const size_t tb0 = ((size_t)t.e * (g.N / kTileN) + tn0) * KT;
        b = static_cast<const uint8_t*>(uniform_ptr(g.b + tb0 * 16 * 1024));
        b_sf = static_cast<const uint8_t*>(uniform_ptr(g.b_sf + tb0 * 256 * 4));
    }
    __device__ __forceinline__ void issue_a(uint8_t* st, int kt, int lane) const {
#pragma unroll
        for (int i = 0; i < A_PW; ++i) {
            const int blk = (i * anw + aw) % L::A_INSTR;
            dma16(a_off[i], a + (size_t)kt * kBK, lds_addr(st + blk * 1024));
        }
        if (sb_wave)  // weight scales [256 columns][4 B] per 256-column block and K-step, contiguous
            dma16((uint32_t)lane * 16, b_sf + ((size_t)sb_blk * KT + kt) * 1024,
                  lds_addr(st + L::A_BYTES + L::B_BYTES + 4 * L::SA_WORDS + sb_blk * 1024));
        else
            dma4(sa_off, a_sf + (size_t)kt * sa_kt, lds_addr(st + L::A_BYTES + L::B_BYTES + sa_blk * 256));
    }
    // weight blocks OFF + i * bnw + bw, i < NB (1 KiB each, 16 per 256 columns).  Instances for routing
    // blocks below the M-tile (block_m < 128: batches with few rows per expert, whose weight tiles serve
    // one or two M-tiles) stream them non-temporally: measured, the decode shape's GEMMs ran 13% faster,
    // prefill's 4% (its combine too, the slot rows staying cached), a 1024-token decode batch 8%.  With
    // block_m >= 128 the hint cost 2-6% where experts span many M-tiles, and choosing it per tile at
    // run time cost 2-3% in the issue path itself.
    template <int NB, int OFF>
    __device__ __forceinline__ void issue_b_blocks(uint8_t* st, int kt, int lane) const {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int blk = OFF + i * bnw + bw;
            const uint8_t* src = b + ((size_t)((blk >> 4) * KT + kt) * 16 + (blk & 15)) * 1024;
            if constexpr (STREAM) dma16_stream((uint32_t)lane * 16, src, lds_addr(st + L::A_BYTES + blk * 1024));
            else dma16((uint32_t)lane * 16, src, lds_addr(st + L::A_BYTES + blk * 1024));
        }
    }
    // the first B_PW * bnw weight blocks
    __device__ __forceinline__ void issue_b(uint8_t* st, int kt, int lane) const {
        issue_b_blocks<B_PW, 0>(st, kt, lane);
    }
};

// ---- fragments of one wave tile (MI x NI MFMA blocks) for one K-step
template <int MI, int NI>
struct Frags {
    v8i a[MI];
    v4i b[NI];
    int sa[MI], sb[NI];
};

// B fragments of all NI blocks and A fragments of blocks [MI0, MI1) of one K-step.
template <int BM, int BN, int MI, int NI, int MI0 = 0, int MI1 = MI, bool WITH_B = true>
__device__ __forceinline__ void read_frags(Frags<MI, NI>& f, const uint8_t* st, int wrow0, int wcol0, int lane) {
    using L = StageLayout<BM, BN>;
    const int gq = lane >> 4;
    const uint8_t* A = st;
    const uint8_t* Bt = st + L::A_BYTES;
    const uint32_t* SA = reinterpret_cast<const uint32_t*>(st + L::A_BYTES + L::B_BYTES);
    const uint32_t* SB = SA + L::SA_WORDS;
    if constexpr (WITH_B) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            const int col = wcol0 + ni * 16 + (lane & 15);
            f.b[ni] = *reinterpret_cast<const v4i*>(Bt + col * (kBK / 2) + ((gq ^ ((col >> 1) & 3)) << 4));
            f.sb[ni] = (int)(SB[col] >> (8 * gq));
        }
    }
#pragma unroll
    for (int mi = MI0; mi < MI1; ++mi) {
        const int row = wrow0 + mi * 16 + (lane & 15);
        const int sw = (row >> 1) & 7;
        const v4i lo = *reinterpret_cast<const v4i*>(A + row * kBK + ((gq ^ sw) << 4));
        const v4i hi = *reinterpret_cast<const v4i*>(A + row * kBK + (((4 + gq) ^ sw) << 4));
        f.a[mi] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        f.sa[mi] = (int)(SA[row] >> (8 * gq));
    }
}

// MFMAs of A blocks [MI0, MI1) against all B blocks; FIRST starts the accumulators from zero
// (the instruction's C operand is the inline constant 0, so no register clearing is needed).
template <int MI, int NI, int MI0 = 0, int MI1 = MI, bool FIRST = false>
__device__ __forceinline__ void mfma_blocks(v4f (&acc)[MI][NI], const Frags<MI, NI>& f) {
#pragma unroll
    for (int mi = MI0; mi < MI1; ++mi) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            const v8i b = v8i{f.b[ni][0], f.b[ni][1], f.b[ni][2], f.b[ni][3], 0, 0, 0, 0};
            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                f.a[mi], b, FIRST ? v4f{0.f, 0.f, 0.f, 0.f} : acc[mi][ni], 0, 4, 0, f.sa[mi], 0, f.sb[ni]);
        }
    }
}
template <int MI, int NI, int MI0 = 0, int MI1 = MI>
__device__ __forceinline__ void mfma_step(v4f (&acc)[MI][NI], const Frags<MI, NI>& f, bool first) {
    if (first) mfma_blocks<MI, NI, MI0, MI1, true>(acc, f);
    else mfma_blocks<MI, NI, MI0, MI1, false>(acc, f);
}

// ---- epilogues: straight from the accumulators to global memory.
// wrow0: the wave's first row within the tile; gcol0: its first global output
// column (a multiple of 64).  The weight tiling permutes columns so that, in
// a 64-column group, MFMA blocks k and k + 2 (k = 0, 1; ni % 4) give lane l
// the gate and the up row of channel 2*(l & 15) + k of the group's 32 SwiGLU
// channels (Linear1: a lane holds both inputs of its two adjacent outputs),
// and in a 128-column span block b = 0..7 gives lane l output 8*(l & 15) + b
// of the span (Linear2).
// PARTIAL: tiles may end before row BM (M-tiles span several routing blocks);
// otherwise every tile has BM valid rows and the row checks compile away.
// COHERENT: the stores are device-scope (sc1) stores, complete at device scope
// once vmcnt has drained (the fused launch hands these rows to other XCDs).
// Linear1 epilogue variants: kEpiFast (hardware exp2/rcp, no clamp; the default), kEpiClamp (the same
// with the activation clamp), kEpiExact (accurate expf and IEEE division, clamp if the limit is > 0).
constexpr int kEpiFast = 0, kEpiClamp = 1, kEpiExact = 2;

template <int BM, int MI, int NI, bool PARTIAL, bool COHERENT, int EPI>
__device__ __forceinline__ void epilogue_linear1(const v4f (&acc)[MI][NI], const GemmArgs& g, int m0, int rows,
                                                 int wrow0, int gcol0, const float* row_w, const int* row_tok,
                                                 int lane) {
    static_assert(NI == 4 || NI == 8, "a wave owns one or two 64-column groups");
    constexpr int NG = NI / 4;              // 64-column groups: 32 channels, one UE8M0 scale per row
    constexpr int V = 4 * NG;               // (group, row) maxima per lane and 16-row block
    constexpr int VSHIFT = V == 8 ? 1 : 2;  // lane j computes the scale of (group, row) j >> VSHIFT
    lane = fresh_lane();                    // per-lane values derived here are not kept across the K-loop
    const int j = lane & 15;
    const int own = j >> VSHIFT;
    const int own_grp = own >> 2, own_i = own & 3;
    const int row_base = (lane & 0x30) * 4;  // ds_bpermute byte address of lane 0 of this DPP row
    const int n_q = g.N / 2;
    const int ksteps2 = g.N / kTileN;  // Linear2 K-steps (128 channels each)
    constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        const int row0 = wrow0 + mi * 16 + 4 * (lane >> 4);  // the lane's rows are row0 .. row0 + 3
        float p[NG][4][2];  // silu(gate) * up of channels 2j and 2j + 1 per group and row
        uint32_t m[V];      // max |p| of each (group, row), as bit patterns
#pragma unroll
        for (int grp = 0; grp < NG; ++grp)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    // gate (block k) and up (block k + 2) rounded to BF16 together, widened back to FP32
                    const uint32_t gu = pack_bf16(acc[mi][grp * 4 + k][i], acc[mi][grp * 4 + 2 + k][i]);
                    float gv = __uint_as_float(gu << 16);
                    float uv = __uint_as_float(gu & 0xFFFF0000u);
                    if (EPI == kEpiClamp || (EPI == kEpiExact && g.swiglu_limit > 0.0f)) {  // activation clamp
                        gv = fminf(gv, g.swiglu_limit);
                        uv = fminf(fmaxf(uv, -g.swiglu_limit), g.swiglu_limit);
                    }
                    // silu(g) = g / (1 + 2^(-g log2 e)) with the hardware exp2 and reciprocal, or with
                    // the accurate expf and IEEE division
                    const float s = EPI == kEpiExact
                                        ? gv / (1.0f + expf(-gv))
                                        : gv * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-gv * kLog2e));
                    p[grp][i][k] = s * uv;
                }
                m[grp * 4 + i] = __float_as_uint(fmaxf(fabsf(p[grp][i][0]), fabsf(p[grp][i][1])));
            }
        // The output is h = p * w (w: the row's top-k weight, 0 on padding rows).  Rounding is
        // monotonic, so max |fl(p w)| = fl(|w| max |p|): the scale comes from the unweighted maximum,
        // and since the requant factor 2^-s is a power of two, fl(fl(p w) 2^-s) = fl(p fl(w 2^-s)).
        const float amax_p = row_max16<V>(m, j);
        const int own_row = row0 + own_i;
        const float wgt = row_tok[own_row] >= 0 ? row_w[own_row] : 0.0f;
        const int code = requant_code(amax_p * fabsf(wgt));
        const float factor = wgt * pow2_neg(code);
        // 32-bit offsets from uniform bases (cap * I < 2^31 is checked on the host)
        if ((j & ((1 << VSHIFT) - 1)) == 0 && (!PARTIAL || own_row < rows)) {
            const int gcol = gcol0 + own_grp * 64;  // first Z column of the 32-channel group
            // Linear2 K-step = 256-column block of Z, byte = 64-column group within it
            uint8_t* sp = g.out_sf + tile_scale_offset<BM, PARTIAL>(m0, own_row, ksteps2, gcol / kTileN, g.bm, g.bm_shift) +
                          (uint32_t)((gcol % kTileN) / 64);
            if constexpr (COHERENT) __hip_atomic_store(sp, (uint8_t)code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else *sp = (uint8_t)code;
        }
#pragma unroll
        for (int grp = 0; grp < NG; ++grp)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // the factor of (grp, row i) from the first lane that computed it
                const float f = __int_as_float(
                    __builtin_amdgcn_ds_bpermute(row_base + ((grp * 4 + i) << VSHIFT) * 4, __float_as_int(factor)));
                const int q = __builtin_amdgcn_cvt_pk_fp8_f32(p[grp][i][0] * f, p[grp][i][1] * f, 0, false);
                const int row_local = row0 + i;
                if (!PARTIAL || row_local < rows) {
                    const uint32_t row = (uint32_t)(m0 + row_local);
                    uint16_t* qp = reinterpret_cast<uint16_t*>(
                        g.out_q + (row * (uint32_t)n_q + (uint32_t)((gcol0 + grp * 64) / 2 + 2 * j)));
                    if constexpr (COHERENT)
                        __hip_atomic_store(qp, (uint16_t)q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    else *qp = (uint16_t)q;
                }
            }
    }
}

template <int BM, int MI, int NI, bool PARTIAL>
__device__ __forceinline__ void epilogue_linear2(const v4f (&acc)[MI][NI], const GemmArgs& g, int m0, int rows,
                                                 int wrow0, int gcol0, const int* row_tok, int lane) {
    static_assert(NI == 4 || NI == 8, "a wave owns half or all of a 128-column span");
    // W2's tiling puts output column 128S + 8j + b in block b of span S, lane j: a lane's NI blocks are
    // NI adjacent outputs starting at this column (16 bytes for a whole span, 8 for half of one)
    const uint32_t col0 = (uint32_t)((gcol0 & ~127) + 8 * (lane & 15) + ((gcol0 & 127) >> 4));
    // the tile's first row is added to the base in 64 bits (uniform: cap * H * 2 may pass 2^32),
    // the lane's offset inside the tile in 32 bits
    uint8_t* out = reinterpret_cast<uint8_t*>(g.out_bf16) + (size_t)(uint32_t)m0 * (uint32_t)g.N * 2u;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row_local = wrow0 + mi * 16 + 4 * (lane >> 4) + i;
            if ((PARTIAL && row_local >= rows) || row_tok[row_local] < 0) continue;  // padding rows are never read
            const uint32_t off = ((uint32_t)row_local * (uint32_t)g.N + col0) * 2u;
            if constexpr (NI == 8) {
                *reinterpret_cast<uint4*>(out + off) =
                    uint4{pack_bf16(acc[mi][0][i], acc[mi][1][i]), pack_bf16(acc[mi][2][i], acc[mi][3][i]),
                          pack_bf16(acc[mi][4][i], acc[mi][5][i]), pack_bf16(acc[mi][6][i], acc[mi][7][i])};
            } else {
                *reinterpret_cast<uint2*>(out + off) =
                    uint2{pack_bf16(acc[mi][0][i], acc[mi][1][i]), pack_bf16(acc[mi][2][i], acc[mi][3][i])};
            }
        }
}

template <int BM, int MI, int NI, bool L1, bool PARTIAL, bool COHERENT = false, int EPI = kEpiFast>
__device__ __forceinline__ void epilogue(const v4f (&acc)[MI][NI], const GemmArgs& g, const TileId& t, int wrow0,
                                         int gcol0, const float* row_w, const int* row_tok, int lane) {
    if constexpr (L1)
        epilogue_linear1<BM, MI, NI, PARTIAL, COHERENT, EPI>(acc, g, t.m, t.rows, wrow0, gcol0, row_w, row_tok,
                                                             lane);
    else epilogue_linear2<BM, MI, NI, PARTIAL>(acc, g, t.m, t.rows, wrow0, gcol0, row_tok, lane);
}

template <int BM, bool L1>
__device__ __forceinline__ void load_row_tables(const GemmArgs& g, const TileId& tl, float* row_w, int* row_tok,
                                                int tid) {
    if (tid < BM) {
        const int t = tid < tl.rows ? g.row_token[tl.m + tid] : -1;
        row_tok[tid] = t;
        if (L1) row_w[tid] = t >= 0 ? g.topk_w[(size_t)t * g.topk + g.row_topk[tl.m + tid]] : 0.0f;
    }
    __syncthreads();
}

// Tile variants of the kernels.  kTileFull: every tile is one routing block of BM rows.  The other two
// cut an expert's rows into tiles of up to BM rows, the last one ending at its last hit: kTileShortStream for
// routing blocks below the M-tile (batches with few rows per expert, whose weight tiles serve one or two
// M-tiles: the weights are streamed with the non-temporal hint, see issue_b_blocks), kTileShortCached for
// routing blocks above it (192 rows: experts span many M-tiles, which reuse the weight tiles from the
// caches, where the hint measured 2-6% slower).
constexpr int kTileFull = 0, kTileShortStream = 1, kTileShortCached = 2;
template <int TV>
constexpr bool kPartial = TV != kTileFull;
template <int BM, int TV>
constexpr bool kStream = BM == 16 || TV == kTileShortStream;

// ============================================================================
// 256-column tiles: one group of 4 waves; per K-step wait, read, multiply.
template <int BM>
struct Cfg4 {
    using L = StageLayout<BM, 256>;
    static constexpr int WM = BM >= 128 ? 2 : 1;  // wave grid rows
    static constexpr int WN = 4 / WM;
    static constexpr int WTM = BM / WM;
    static constexpr int WTN = 256 / WN;
    static_assert(WTN % 64 == 0, "a wave must own whole 64-column requant groups");
    static constexpr int MI = WTM / 16, NI = WTN / 16;
    static constexpr int A_PW = L::A_INSTR >= 4 ? L::A_INSTR / 4 : 1;
    static constexpr int B_PW = L::B_INSTR / 4;
    static constexpr int D = A_PW + 1 + B_PW;  // DMA instructions per wave per stage
    static_assert(2 * D < 64, "vmcnt range");
};

template <int BM, bool L1, int TV, int EPI>
__global__ __launch_bounds__(256, 1) void gemm4_kernel(GemmArgs g) {
    constexpr bool PARTIAL = kPartial<TV>;
    using C = Cfg4<BM>;
    using L = typename C::L;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[L::NS * L::STAGE];
    __shared__ float row_w[BM];
    __shared__ int row_tok[BM];

    if (L1 && g.status && blockIdx.x == 0 && threadIdx.x == 0) *g.status = 0u;
    TileId t;
    if (!tile_of_block(g, 256, t)) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int KT = g.K / kBK;
    load_row_tables<BM, L1>(g, t, row_w, row_tok, tid);

    StageDma<BM, 256, C::A_PW, C::B_PW, kStream<BM, TV>> dma;
    dma.init_a(g, t.m, t.rows, row_tok, L1, w, 4);
    dma.init_b(g, t, w, 4);
    auto issue = [&](int kt) {
        uint8_t* st = smem + (kt % L::NS) * L::STAGE;
        dma.issue_a(st, kt, lane);
        dma.issue_b(st, kt, lane);
    };

    const int wrow0 = (w / C::WN) * C::WTM, wcol0 = (w % C::WN) * C::WTN;
    v4f acc[C::MI][C::NI];
#pragma unroll
    for (int s = 0; s < L::NS - 1; ++s)
        if (s < KT) issue(s);
    for (int kt = 0; kt < KT; ++kt) {
        wait_stages_and_barrier<C::D>(min(L::NS - 2, KT - 1 - kt));  // stage kt landed; kt-1 fully read
        if (kt + L::NS - 1 < KT) issue(kt + L::NS - 1);
        Frags<C::MI, C::NI> f;
        read_frags<BM, 256>(f, smem + (kt % L::NS) * L::STAGE, wrow0, wcol0, lane);
        mfma_step(acc, f, kt == 0);
    }
    epilogue<BM, C::MI, C::NI, L1, PARTIAL, false, EPI>(acc, g, t, wrow0, t.n * 256 + wcol0, row_w, row_tok, lane);
}

// ============================================================================
// 512-column tiles: two groups of 4 waves in ping-pong, persistent over a
// run of tiles.
//
// A workgroup owns tiles L_j = first + j * nslots (j < ntiles) of its XCD's
// contiguous chunk of the tile list and walks their K-steps as one sequence
// gs = 0 .. S-1 (S = ntiles * KT; tile j = gs / KT, K-step gs % KT), so the
// operand ring runs on across tile boundaries and the next tile's first
// stages load while the current one finishes.
//
// One workgroup barrier B_gs per K-step.  Between B_gs and B_gs+1 group 0
// issues its share of stage gs + NS - 1, reads stage gs and multiplies it,
// while group 1 first multiplies stage gs - 1 (read before B_gs), then
// issues its share of stage gs + NS - 1 and reads stage gs.  So each group's
// DMA issue and LDS reads run while the other group's MFMAs occupy the
// SIMD's matrix core, with no barrier between the two halves: the halves
// find their own balance, and a barrier costs a few hundred cycles.
//   * before B_gs each wave waits for its own share of stage gs (vmcnt), so
//     stage gs is whole after B_gs;
//   * stage gs + NS - 1 reuses the buffer of stage gs - 1, whose reads all
//     fall before B_gs: each wave waits for its LDS reads (lgkmcnt(0))
//     before every barrier.
// Both groups pass the same S barriers; group 1 multiplies stage S - 1
// after the last one.  Group 1 runs the epilogue of a tile right after its
// last MFMAs of that tile (half a step after group 0, overlapping group 0's
// next issue, reads and MFMAs).  Group 0 runs it after the next barrier,
// before its next MFMAs, so it overlaps group 1's MFMAs instead of holding
// group 1 at the barrier (measured: Linear2 1-1.3% and Linear1 ~1%
// faster).
//
// Per-tile tables reach LDS through the same DMA stream, a fixed number of
// extra instructions per wave per stage so the vmcnt arithmetic stays exact:
// group 0 loads the list entry of tile ci + 2 into desc[(ci + 2) % 3];
// group 1 loads the row tokens and top-k slots of tile ci + 1 into
// meta[(ci + 1) % 3] (ci = the tile being multiplied; between tile changes
// the same load repeats, rewriting identical bytes).  For Linear1 group 1
// also gathers the top-k weights of a tile through those tables into
// wts[.. % 3], once, with the tile's first stage (a 64-line scatter per
// instruction, too costly to repeat every stage); its vmcnt waits count that
// instruction where it falls.  With KT >= 2 (NS - 1) K-steps per tile
// every table has landed before it is read: a list entry by the time its
// rows are fetched, the rows by the time the tile's first stage is issued,
// the weights by the time the tile's multiplication starts.  Below that the
// kernel runs one tile per workgroup.
//
// Fused launch (Linear1 and Linear2 in one kernel: the single-launch
// schedule of the reading notes, where Linear2 blocks wait on arrival marks
// set by the Linear1 epilogue).  Each workgroup runs the loop above over its
// Linear1 tiles, then again, after a barrier, over its Linear2 tiles.  When
// both groups have stored the h rows of a Linear1 tile (each wave fencing
// its stores at device scope), one lane stores the launch's epoch into that
// tile's flag.  In the Linear2 run group 1 also loads the flags of tile
// ci + 1's M-tile with its row tables (gate[.. % 3], read device-coherent),
// and before it issues the activation DMA of K-step kt it checks that the
// flag of Linear1 N-tile kt / 2, the one that wrote those 128 channels,
// holds the epoch, else sleeps and loads the flags again.  A workgroup's own
// Linear1 tiles are all flagged before its Linear2 run starts, every
// workgroup runs its Linear1 tiles first, and the grid is at most one
// workgroup per CU, all resident: every awaited tile is being computed.  A
// Linear2 K-step reads only channels whose Linear1 tile is done, and no XCD
// reads those lines earlier in the launch (a row's 128 channels of one
// K-step are one 128-byte line of h_q; its scale words of K-steps 2m and
// 2m + 1, which can share a line when block_m is 16, come from the same
// Linear1 tile), so plain loads see the stored values.  After kGateSpins polls
// the wait gives up and sets the status word instead of hanging (the tile
// then computes on rows that may be unfinished, and the combine, which reads
// the word, writes NaN over all of y).
//
// The epoch is the value of a per-workspace counter that a one-thread kernel
// advances ahead of every fused launch, eager or recorded into a graph, and
// that nothing writes during the launch; successive launches on one
// workspace therefore stamp distinct values for 2^32 launches.  It is passed
// through a fixed bijection so that a workspace filled with one byte value
// (counter and flags alike) does not start with matching flags.
template <int BM, bool L1, bool FUSED>
struct CfgPP {
    using L = StageLayout<BM, 512>;
    static constexpr bool SPLIT_ROWS = BM == 128;  // the groups split the rows, else the columns
    static constexpr int WTM = SPLIT_ROWS ? 64 : BM;
    static constexpr int WTN = SPLIT_ROWS ? 128 : 64;
    static constexpr int MI = WTM / 16, NI = WTN / 16;
    // The weight blocks are split between the groups so that their read phases, which carry the
    // DMA issue, are about as long: group 0 issues B0_PW weight blocks per wave and the list
    // entry; group 1 the activation rows, one scale block per wave (activation or weight
    // scales), B1_PW weight blocks per wave and the row tables.  (Measured on tp_slice: without any weight DMA the
    // GEMMs ran 13-18% faster, without any row DMA no faster, so the weights-only group was
    // the one the other waited for.)
    static constexpr int A_PW = L::A_INSTR >= 4 ? L::A_INSTR / 4 : 1;
    static constexpr int B_PW = L::B_INSTR / 4;
    static constexpr int B1_PW = A_PW >= 4 ? B_PW / 4 : B_PW / 2;
    static constexpr int B0_PW = B_PW - B1_PW;
    static constexpr int D0 = B0_PW + 1;
    static constexpr bool GATED = FUSED && !L1;  // + the Linear1 flags of the next tile
    static constexpr int D1 = A_PW + B1_PW + 1 + 1 + (GATED ? 1 : 0);  // + 1 on the first stage of each tile (Linear1)
    static constexpr int MIN_KT_PERSISTENT = 2 * (L::NS - 1);
    static_assert(2 * D0 < kNoVmWait && 2 * D1 + 1 < kNoVmWait, "vmcnt range");
    static_assert(BM <= 128, "row tables hold 128 rows");
};
constexpr int kTableSlots = 3;
constexpr int kGateSpins = 1 << 18;  // flag polls (a few us each) before a Linear2 tile gives up

// Completion flags of a fused launch.
struct FusedSync {
    uint32_t* flags;   // one word per Linear1 tile, [M-tile][Linear1 N-tile]
    uint32_t* status;  // set to 1 if a Linear2 tile stopped waiting
    uint32_t epoch;    // value of a set flag in this launch
    int nt1;           // Linear1 N-tiles
};

// LDS of the persistent kernels.
template <int BM>
struct PPShared {
    __attribute__((aligned(1024))) uint8_t smem[StageLayout<BM, 512>::NS * StageLayout<BM, 512>::STAGE];
    int desc[kTableSlots][64];       // words 0-3: the tile's list entry
    int meta[kTableSlots][256];      // [0, 128): row tokens; [128, 256): top-k slots
    float wts[kTableSlots][128];     // Linear1: top-k weights of the rows
    uint32_t gate[kTableSlots][64];  // fused Linear2: the Linear1 flags of the tile's M-tile
};

// The tiles of one persistent run, in order: j < n_a: first_a + j * stride_a,
// then first_b + (j - n_a) * stride_b.
struct TileSeq {
    int first_a, n_a, stride_a, first_b, stride_b, n;
    __device__ __forceinline__ int index(int j) const {
        return j < n_a ? first_a + j * stride_a : first_b + (j - n_a) * stride_b;
    }
};

// One persistent run over the tiles `seq` of g's list.
template <int BM, bool L1, int TV, bool FUSED, int EPI>
__device__ __forceinline__ void pp_run(const GemmArgs& g, const FusedSync& sync, const TileSeq& seq,
                                       PPShared<BM>& sh) {
    constexpr bool PARTIAL = kPartial<TV>;
    const int ntiles = seq.n;
    using C = CfgPP<BM, L1, FUSED>;
    using L = typename C::L;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = w >> 2, wq = w & 3;
    const int KT = g.K / kBK;
    const int S = ntiles * KT;
    auto tile_entry = [&](int j) {
        return static_cast<const int32_t*>(uniform_ptr(g.tiles + kTileWords * seq.index(min(j, ntiles - 1))));
    };

    // ---- table loads (one DMA instruction per wave)
    auto load_desc = [&](int j) {  // group 0
        j = min(j, ntiles - 1);
        dma4((uint32_t)min(fresh_lane(), kTileWords - 1) * 4, tile_entry(j), lds_addr(&sh.desc[j % kTableSlots][0]));
    };
    // fused Linear2: the Linear1 flags of tile t's M-tile, read device-coherent (sc1: other
    // workgroups, possibly on other XCDs, store them)
    auto load_flags = [&](int j, const TileId& t) {
        asm volatile("global_load_lds_dword %0, %1 sc1"
                     ::"v"((uint32_t)(t.mt * sync.nt1 + min(fresh_lane(), sync.nt1 - 1)) * 4u), "s"(sync.flags),
                       "{m0}"(lds_addr(&sh.gate[j % kTableSlots][0]))
                     : "memory");
    };
    // rows past the tile's valid count load whatever the tables hold there (the
    // tables reserve slack rows past the last block); every reader masks them
    auto load_meta = [&](int j, const TileId& t) {  // group 1; t = tile j
        j = min(j, ntiles - 1);
        const int part = wq >> 1, half = wq & 1;
        const int row = min(half * 64 + fresh_lane(), BM - 1);
        const int32_t* src = (part == 1 ? g.row_topk : g.row_token) + t.m;
        dma4((uint32_t)row * 4, src, lds_addr(&sh.meta[j % kTableSlots][part * 128 + half * 64]));
        if constexpr (C::GATED) load_flags(j, t);
    };
    auto read_entry = [&](int j, TileId& t) {
        j = min(j, ntiles - 1);
        const int* d = sh.desc[j % kTableSlots];
        t.m = __builtin_amdgcn_readfirstlane(d[0]);
        const int b = __builtin_amdgcn_readfirstlane(d[1]);
        t.n = b >> 16;
        t.e = b & 0xFFFF;
        t.rows = PARTIAL ? __builtin_amdgcn_readfirstlane(d[2]) : BM;
        t.mt = FUSED ? __builtin_amdgcn_readfirstlane(d[3]) : 0;
    };

    const int wrow0 = C::SPLIT_ROWS ? grp * C::WTM : 0;
    const int wcol0 = C::SPLIT_ROWS ? wq * C::WTN : grp * 256 + wq * C::WTN;
    v4f acc[C::MI][C::NI];  // set by the first K-step of every tile
    TileId ct;              // tile being multiplied

    // ---- prologue: list entries of tiles 0 and 1, then the rows of tile 0
    if (grp == 0) load_desc(wq & 1);
    wait_and_barrier<0>();
    TileId t0;
    read_entry(0, t0);
    if (grp == 1) load_meta(0, t0);
    wait_and_barrier<0>();

    if (grp == 0) {
        StageDma<BM, 512, 1, C::B0_PW, kStream<BM, TV>> dma;
        dma.init_b(g, t0, wq, 4);
        // stage s (and the table load that rides with it) for compute step gs = s - (NS - 1)
        auto issue = [&](int s) {
            if (s % KT == 0 && s > 0) {
                TileId t;
                read_entry(s / KT, t);
                dma.init_b(g, t, wq, 4);
            }
            dma.issue_b(sh.smem + (s % L::NS) * L::STAGE, s % KT, lane);
            load_desc(max(s - (L::NS - 1), 0) / KT + 2);
        };
#pragma unroll
        for (int s = 0; s < L::NS - 1; ++s)
            if (s < S) issue(s);
        // the epilogue of a finished tile runs after the next barrier (it then overlaps group 1's MFMAs
        // instead of holding group 1 at the barrier), before this group's next MFMAs
        bool pending = false;
        TileId pt;
        int pci = 0;
        auto deferred_epilogue = [&]() {
            if (pending) {
                epilogue<BM, C::MI, C::NI, L1, PARTIAL, FUSED, EPI>(acc, g, pt, wrow0, pt.n * 512 + wcol0,
                                                               sh.wts[pci % kTableSlots],
                                                               sh.meta[pci % kTableSlots], lane);
                if constexpr (FUSED && L1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // stores complete
            }
            pending = false;
        };
        for (int gs = 0, kt = 0, ci = 0; gs < S; ++gs) {
            wait_stages_and_barrier<C::D0>(min(L::NS - 2, S - 1 - gs));  // B_gs
            deferred_epilogue();
            if (kt == 0) read_entry(ci, ct);
            if (gs + L::NS - 1 < S) issue(gs + L::NS - 1);
            Frags<C::MI, C::NI> f;
            read_frags<BM, 512>(f, sh.smem + (gs % L::NS) * L::STAGE, wrow0, wcol0, lane);
            mfma_step(acc, f, kt == 0);
            if (++kt == KT) {
                pending = true;
                pt = ct;
                pci = ci;
                kt = 0;
                ++ci;
            }
        }
        deferred_epilogue();
        if constexpr (FUSED) __syncthreads();  // B_S
    } else {
        StageDma<BM, 512, C::A_PW, 1, kStream<BM, TV>> dma;
        // fused Linear2: before the activation DMA of K-step kt of tile j, wait until the Linear1 tile
        // that wrote those channels of t's rows is done.  Linear2 K-step kt reads h channels
        // [128 kt, 128 kt + 128), which Linear1 N-tile kt / 2 (256 SwiGLU channels, 512 gate/up
        // columns) produced, so a K-step needs one flag, not the whole M-tile's (the reading notes'
        // per-K-block gating).  The flags of the M-tile came with the row tables.  At a tile's first
        // stage all of them are looked at once; when they are all set (the usual case: an M-tile's
        // Linear1 tiles run side by side and finish together) the tile's later stages check nothing.
        // Otherwise each K-step waits for its own flag: while it is not set, sleep and load the flags
        // again (the wait for that load drains this wave's DMA queue, which only makes the later
        // vmcnt waits conservative), and stop checking once all are set.
        bool gate_all = false;  // every flag of the issuing tile's M-tile holds the epoch
        auto gate_open = [&](int j, const TileId& t, int kt) {
            if constexpr (C::GATED) {
                const uint32_t* fl = sh.gate[j % kTableSlots];
                if (kt == 0) gate_all = false;
                if (gate_all) return;
                const int need = kt >> 1;
                for (int it = 0;; ++it) {
                    const int l = fresh_lane();
                    const bool ok = l >= sync.nt1 || fl[l] == sync.epoch;
                    if (__builtin_amdgcn_ballot_w64(!ok) == 0) {
                        gate_all = true;
                        return;
                    }
                    if (__builtin_amdgcn_readfirstlane(fl[need]) == sync.epoch) return;
                    if (it == kGateSpins) {
                        if (l == 0) __hip_atomic_store(sync.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        return;
                    }
                    __builtin_amdgcn_s_sleep(16);
                    load_flags(j, t);
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                }
            }
        };
        TileId itile = t0;  // tile whose stages are being issued
        dma.init_a(g, t0.m, t0.rows, sh.meta[0], L1, wq, 4);
        dma.init_b(g, t0, wq, 4);
        TileId tn;  // tile whose rows the table load fetches
        read_entry(1, tn);
        // Linear1: byte offset into topk_w of this lane's row of the issued tile
        auto weight_offset = [&](int j, int rows) {
            const int w_row = min((wq & 1) * 64 + fresh_lane(), BM - 1);
            const int* mt = sh.meta[j % kTableSlots];
            const int t = w_row < rows ? mt[w_row] : -1;
            return t >= 0 ? (uint32_t)(t * g.topk + mt[128 + w_row]) * 4u : 0u;
        };
        uint32_t w_off = L1 ? weight_offset(0, t0.rows) : 0u;
        auto issue = [&](int s) {
            if (s % KT == 0 && s > 0) {
                read_entry(s / KT, itile);
                dma.init_a(g, itile.m, itile.rows, sh.meta[(s / KT) % kTableSlots], L1, wq, 4);
                dma.init_b(g, itile, wq, 4);
                if (L1) w_off = weight_offset(s / KT, itile.rows);
            }
            gate_open(s / KT, itile, s % KT);
            dma.issue_a(sh.smem + (s % L::NS) * L::STAGE, s % KT, lane);
            dma.template issue_b_blocks<C::B1_PW, 4 * C::B0_PW>(sh.smem + (s % L::NS) * L::STAGE, s % KT, lane);
            load_meta(max(s - (L::NS - 1), 0) / KT + 1, tn);
            if (L1 && s % KT == 0)
                dma4(w_off, g.topk_w, lds_addr(&sh.wts[(s / KT) % kTableSlots][(wq & 1) * 64]));
        };
        // does a stage in (s, s + n] start a tile (and so carry the weight gather)?
        auto starts_tile = [&](int s, int n) { return L1 && n > 0 && ((s % KT) + n >= KT) ? 1 : 0; };
        // fused Linear1: the flag of a finished tile is stored after the next barrier, when both
        // groups' stores of that tile are fenced
        bool signal = false;
        TileId done;
        auto store_flag = [&]() {
            if (signal && w == 4 && lane == 0)
                __hip_atomic_store(sync.flags + done.mt * sync.nt1 + done.n, sync.epoch, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            signal = false;
        };
#pragma unroll
        for (int s = 0; s < L::NS - 1; ++s)
            if (s < S) issue(s);
        // step gs - 1's product and epilogue, then the issue and the fragment reads of step gs
        Frags<C::MI, C::NI> f;
        int kt = 0, ci = 0;
        auto multiply = [&]() {
            mfma_step(acc, f, kt == 0);
            if (++kt == KT) {
                epilogue<BM, C::MI, C::NI, L1, PARTIAL, FUSED, EPI>(acc, g, ct, wrow0, ct.n * 512 + wcol0,
                                                               sh.wts[ci % kTableSlots], sh.meta[ci % kTableSlots],
                                                               lane);
                if constexpr (FUSED && L1) {
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // stores complete
                    signal = true;
                    done = ct;
                }
                kt = 0;
                ++ci;
            }
        };
        for (int gs = 0; gs < S; ++gs) {
            {  // B_gs
                const int n = min(L::NS - 2, S - 1 - gs);
                wait_stages_and_barrier<C::D1>(n, starts_tile(gs, n));
            }
            if constexpr (FUSED && L1) store_flag();
            if (gs > 0) multiply();
            if (kt == 0) {
                read_entry(ci, ct);
                read_entry(ci + 1, tn);
            }
            if (gs + L::NS - 1 < S) issue(gs + L::NS - 1);
            read_frags<BM, 512>(f, sh.smem + (gs % L::NS) * L::STAGE, wrow0, wcol0, lane);
        }
        multiply();  // stage S - 1 (S > 0: a run has at least one tile)
        if constexpr (FUSED) {
            __syncthreads();  // B_S
            if constexpr (L1) store_flag();
        }
    }
}

// Round-robin share of an XCD's list range [begin, end): tiles begin + slot + j * nslots.
__device__ __forceinline__ TileSeq round_robin(int begin, int end, int slot, int nslots) {
    const int first = begin + slot;
    const int n = first < end ? (end - first + nslots - 1) / nslots : 0;
    return TileSeq{first, n, nslots, 0, 1, n};
}

template <int BM, bool L1, int TV, int EPI>
__global__ __launch_bounds__(512, 1) void gemm_pp_kernel(GemmArgs g) {
    __shared__ PPShared<BM> sh;
    if (L1 && g.status && blockIdx.x == 0 && threadIdx.x == 0) *g.status = 0u;
    int begin, end;
    xcd_chunk(g, g.N / 512, blockIdx.x % kNumXcd, begin, end);
    const TileSeq seq = round_robin(begin, end, blockIdx.x / kNumXcd, gridDim.x / kNumXcd);
    if (seq.n == 0) return;
    pp_run<BM, L1, TV, false, EPI>(g, FusedSync{}, seq, sh);
}

struct FusedArgs {
    GemmArgs g1, g2;  // Linear1, Linear2
    FusedSync sync;   // sync.epoch is set on the device from epoch_word
    // the workspace's launch counter, advanced by fused_prepare_kernel ahead of this launch
    const uint32_t* epoch_word;
};

// Flag value of the launch whose counter value is w: an odd-multiplier bijection of the 32-bit counter
// (distinct counters give distinct values) followed by a constant xor, so that a counter and flags
// holding the same fill pattern do not match (0x00.., 0x5A.., 0xAB.., 0xFF.. were checked).
__device__ __forceinline__ uint32_t flag_value(uint32_t w) { return (w * 0x9E3779B1u) ^ 0x6C8E9CF5u; }

// Runs (one thread) ahead of every fused launch on the same stream: advances the workspace's launch
// counter, so that the launch stamps flags no earlier launch on the workspace stamped, and clears the
// status word, which then reports on this launch only.
__global__ void fused_prepare_kernel(uint32_t* epoch_word, uint32_t* status) {
    if (threadIdx.x == 0) {
        const uint32_t v = __hip_atomic_load(epoch_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(epoch_word, v + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(status, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Linear1 then Linear2 in one launch.  Each XCD runs the Linear1 and then the Linear2 tiles of its
// M-tiles.  Its Linear1 tiles go round-robin to its workgroups, so the first r1 slots run one tile
// more than the others ("light" workgroups, L of them).  While the others finish that tile, the
// light workgroups run the first L * d Linear2 tiles (d = Linear2 tiles per Linear1 tile of time,
// from the K-steps; the list runs M-tile by M-tile, so these need the M-tiles the first Linear1
// round computed); the rest go round-robin to all workgroups.
template <int BM, int TV, int EPI>
__global__ __launch_bounds__(512, 1) void gemm_fused_kernel(FusedArgs fa) {
    __shared__ PPShared<BM> sh;
    const int nslots = gridDim.x / kNumXcd, xcd = blockIdx.x % kNumXcd, slot = blockIdx.x / kNumXcd;
    FusedSync sync = fa.sync;
    // every workgroup reads the same counter value: nothing in this launch writes the word
    sync.epoch = __builtin_amdgcn_readfirstlane(
        flag_value(__hip_atomic_load(fa.epoch_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
    int b1, e1, b2, e2;
    xcd_chunk(fa.g1, fa.g1.N / 512, xcd, b1, e1);
    xcd_chunk(fa.g2, fa.g2.N / 512, xcd, b2, e2);
    const TileSeq s1 = round_robin(b1, e1, slot, nslots);
    if (s1.n > 0) pp_run<BM, true, TV, true, EPI>(fa.g1, sync, s1, sh);
    wait_and_barrier<0>();  // the Linear1 run's table loads have landed before the tables are reused

    const int r1 = (e1 - b1) % nslots, nl = r1 > 0 ? nslots - r1 : 0;  // light workgroups: slots >= r1
    const int c1 = fa.g1.K / kBK + 1, c2 = fa.g2.K / kBK + 1;            // tile costs in K-steps
    const int d = (2 * c1 + c2) / (2 * c2);
    const int na_all = min(nl * d, e2 - b2);
    TileSeq s2;
    const int li = slot - r1;
    s2.first_a = b2 + li;
    s2.stride_a = max(nl, 1);
    s2.n_a = (r1 > 0 && li >= 0 && li < na_all) ? (na_all - li + nl - 1) / nl : 0;
    s2.first_b = b2 + na_all + slot;
    s2.stride_b = nslots;
    s2.n = s2.n_a + (s2.first_b < e2 ? (e2 - s2.first_b + nslots - 1) / nslots : 0);
    if (s2.n > 0) pp_run<BM, false, TV, true, kEpiFast>(fa.g2, sync, s2, sh);
}

// Compute units of the current device (cached per device).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
        cache[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

// K-steps a tile needs for the persistent ping-pong kernel with M-tile bmg.
int min_kt_persistent(int bmg) {
    switch (bmg) {
        case 16: return CfgPP<16, true, false>::MIN_KT_PERSISTENT;
        case 128: return CfgPP<128, true, false>::MIN_KT_PERSISTENT;
        default: return 1 << 30;
    }
}

int64_t persistent_grid(int64_t all) {
    const int64_t cus = device_cus() / kNumXcd * kNumXcd;  // one workgroup per CU
    return std::max<int64_t>(kNumXcd, std::min(all, cus));
}

template <int BM, bool L1, int TV, int EPI>
hipError_t launch_bm_epi(const GemmArgs& args, int64_t all, hipStream_t stream) {
    if (gemm_bn(args.N) == 512) {
        const int64_t grid = args.K / kBK >= min_kt_persistent(BM) ? persistent_grid(all) : all;
        hipLaunchKernelGGL((gemm_pp_kernel<BM, L1, TV, EPI>), dim3(grid), dim3(512), 0, stream, args);
    } else {
        hipLaunchKernelGGL((gemm4_kernel<BM, L1, TV, EPI>), dim3(all), dim3(256), 0, stream, args);
    }
    return hipGetLastError();
}

// Linear1 epilogue variant of a problem
int epi_of(const GemmArgs& a) { return a.exact_silu ? kEpiExact : a.swiglu_limit > 0.0f ? kEpiClamp : kEpiFast; }

template <int BM, int TV>
void launch_fused(int epi, dim3 grid, dim3 block, hipStream_t stream, const FusedArgs& fa) {
    if (epi == kEpiClamp) hipLaunchKernelGGL((gemm_fused_kernel<BM, TV, kEpiClamp>), grid, block, 0, stream, fa);
    else if (epi == kEpiExact) hipLaunchKernelGGL((gemm_fused_kernel<BM, TV, kEpiExact>), grid, block, 0, stream, fa);
    else hipLaunchKernelGGL((gemm_fused_kernel<BM, TV, kEpiFast>), grid, block, 0, stream, fa);
}

// all: workgroups for one tile each
template <int BM, bool L1, int TV>
hipError_t launch_bm(const GemmArgs& args, int64_t all, hipStream_t stream) {
    if constexpr (L1) {
        switch (epi_of(args)) {
            case kEpiClamp: return launch_bm_epi<BM, true, TV, kEpiClamp>(args, all, stream);
            case kEpiExact: return launch_bm_epi<BM, true, TV, kEpiExact>(args, all, stream);
            default: return launch_bm_epi<BM, true, TV, kEpiFast>(args, all, stream);
        }
    }
    return launch_bm_epi<BM, L1, TV, kEpiFast>(args, all, stream);
}

// Workgroups for one tile each of a GEMM with N columns: every XCD gets the slots of ceil(M-tiles / 8)
// M-tiles (xcd_chunk), for an upper bound on the M-tiles (the padded rows are not known on the host).
int64_t one_tile_grid(const GemmProblem& p, int N) {
    const int64_t mtiles = max_m_tiles(*p.shape);
    return kNumXcd * ((mtiles + kNumXcd - 1) / kNumXcd) * (N / gemm_bn(N));
}

template <bool L1>
hipError_t launch_gemm(const GemmProblem& p, GemmArgs args, hipStream_t stream) {
    const int bm = p.shape->block_m, bmg = gemm_bm(bm);
    const int64_t tiles = one_tile_grid(p, args.N);
    if (tiles == 0) return hipSuccess;
    if (bmg == bm) {
        switch (bmg) {
            case 16: return launch_bm<16, L1, kTileFull>(args, tiles, stream);
            case 128: return launch_bm<128, L1, kTileFull>(args, tiles, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (bmg) {
        case 128:
            if (bm < bmg) return launch_bm<128, L1, kTileShortStream>(args, tiles, stream);
            return launch_bm<128, L1, kTileShortCached>(args, tiles, stream);
        default: return hipErrorInvalidValue;
    }
}

GemmArgs common_args(const GemmProblem& p) {
    GemmArgs a{};
    a.scalars = p.plan->scalars;
    a.row_token = p.plan->row_token;
    a.row_topk = p.plan->row_topk;
    a.topk = p.shape->topk;
    a.bm = p.shape->block_m;
    a.bm_shift = (a.bm & (a.bm - 1)) == 0 ? 31 - __builtin_clz((unsigned)a.bm) : -1;
    a.swiglu_limit = p.shape->swiglu_limit;
    a.exact_silu = p.shape->exact_silu;
    return a;
}

GemmArgs linear1_args(const GemmProblem& p, const uint8_t* x, const uint8_t* x_sf, const float* topk_w,
                      const uint8_t* w1, const uint8_t* w1_sf, uint8_t* h_q, uint8_t* h_sf, uint32_t* status) {
    GemmArgs a = common_args(p);
    a.status = status;
    a.tiles = p.plan->tiles1;
    a.count_idx = 4;
    a.topk_w = topk_w;
    a.a = x; a.a_sf = x_sf; a.b = w1; a.b_sf = w1_sf;
    a.out_q = h_q; a.out_sf = h_sf; a.out_bf16 = nullptr;
    a.K = p.shape->hidden; a.N = 2 * p.shape->intermediate;
    return a;
}

GemmArgs linear2_args(const GemmProblem& p, const uint8_t* h_q, const uint8_t* h_sf, const uint8_t* w2,
                      const uint8_t* w2_sf, uint16_t* yslot) {
    GemmArgs a = common_args(p);
    a.tiles = p.plan->tiles2;
    a.count_idx = 5;
    a.a = h_q; a.a_sf = h_sf; a.b = w2; a.b_sf = w2_sf;
    a.out_q = nullptr; a.out_sf = nullptr; a.out_bf16 = yslot;
    a.K = p.shape->intermediate; a.N = p.shape->hidden;
    return a;
}

}  // namespace

bool fused_supported(const moe_shape& s) {
    const int bmg = gemm_bm(s.block_m);
    const int N1 = 2 * s.intermediate, N2 = s.hidden;
    return gemm_bn(N1) == 512 && gemm_bn(N2) == 512 && N1 / 512 <= 64 &&
           s.hidden / kBK >= min_kt_persistent(bmg) && s.intermediate / kBK >= min_kt_persistent(bmg);
}

int cu_count() { return device_cus(); }

bool forward_one_launch(const moe_shape& s, int cus) {
    if (!fused_supported(s)) return false;
    // M-tiles: each expert's padded rows in tiles of bmg, at most cap / bmg + one partial tile per expert
    const int64_t m_tiles = capacity_rows(s) / gemm_bm(s.block_m) + s.num_experts;
    const int64_t tiles1 = m_tiles * (2 * s.intermediate / 512);
    return tiles1 <= (int64_t)kOneLaunchTilesPerCu * cus;
}

hipError_t launch_expert_ffn(const GemmProblem& p, const uint8_t* x, const uint8_t* x_sf, const float* topk_w,
                             const uint8_t* w1, const uint8_t* w1_sf, uint8_t* h_q, uint8_t* h_sf,
                             const uint8_t* w2, const uint8_t* w2_sf, uint16_t* yslot, uint32_t* flags,
                             uint32_t* status, uint32_t* epoch_word, hipStream_t stream, bool prepared) {
    FusedArgs fa{};
    fa.g1 = linear1_args(p, x, x_sf, topk_w, w1, w1_sf, h_q, h_sf, status);
    fa.g2 = linear2_args(p, h_q, h_sf, w2, w2_sf, yslot);
    if (!fused_supported(*p.shape)) {
        hipError_t e = launch_gemm<true>(p, fa.g1, stream);
        if (e != hipSuccess) return e;
        return launch_gemm<false>(p, fa.g2, stream);
    }
    fa.g1.status = nullptr;  // fused_prepare_kernel clears the word
    fa.sync.flags = flags;
    fa.sync.status = status;
    fa.sync.nt1 = fa.g1.N / 512;
    fa.epoch_word = epoch_word;
    const int64_t tiles = std::max(one_tile_grid(p, fa.g1.N), one_tile_grid(p, fa.g2.N));
    if (tiles == 0) return hipSuccess;
    const dim3 grid((unsigned)persistent_grid(tiles)), block(512);
    const int bm = p.shape->block_m, bmg = gemm_bm(bm);
    const int epi = epi_of(fa.g1);
    // advance the launch counter (eager or recorded alike), so that this launch's flag value is new, and
    // clear the status word: here, or done by the routing kernels just enqueued
    if (!prepared) {
        hipLaunchKernelGGL(fused_prepare_kernel, dim3(1), dim3(64), 0, stream, epoch_word, status);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (bmg == 16) launch_fused<16, kTileFull>(epi, grid, block, stream, fa);
    else if (bm == 128) launch_fused<128, kTileFull>(epi, grid, block, stream, fa);
    else if (bm < 128) launch_fused<128, kTileShortStream>(epi, grid, block, stream, fa);
    else launch_fused<128, kTileShortCached>(epi, grid, block, stream, fa);
    return hipGetLastError();
}

hipError_t launch_linear1(const GemmProblem& p, const uint8_t* x, const uint8_t* x_sf, const float* topk_w,
                          const uint8_t* w1, const uint8_t* w1_sf, uint8_t* h_q, uint8_t* h_sf, uint32_t* status,
                          hipStream_t stream) {
    return launch_gemm<true>(p, linear1_args(p, x, x_sf, topk_w, w1, w1_sf, h_q, h_sf, status), stream);
}

hipError_t launch_linear2(const GemmProblem& p, const uint8_t* h_q, const uint8_t* h_sf, const uint8_t* w2,
                          const uint8_t* w2_sf, uint16_t* yslot, hipStream_t stream) {
    return launch_gemm<false>(p, linear2_args(p, h_q, h_sf, w2, w2_sf, yslot), stream);
}

}  // namespace moe
