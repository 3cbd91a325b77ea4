// Data re-layouts for the grouped GEMMs.
//
// Weights are re-laid once, before any forward (the pages do the same with
// their one-time weight transform: gate/up interleave plus a scale
// transpose for their tensor-memory copy, SymmBuffer page section 7).  The
// tiled layout here makes every 128-wide K-step of a 256-column weight tile
// one contiguous block, already in the order the GEMM keeps it in LDS, so
// the stage loads are fully contiguous 1 KiB DMA transfers:
//
//   data   [E][N/256][K/128][1024 slots of 16 B]; slot p holds the 16 bytes
//          of tile column c = p >> 2, logical chunk q = (p & 3) ^ ((c >> 1) & 3),
//          i.e. bytes [kt*64 + q*16, +16) of that column's packed FP4 row;
//   scales [E][N/256][K/128][256 columns][4 B]: the four UE8M0 bytes of the
//          column for that K-step.
//
// Tile column c of a 256-column block holds weight row nt*256 + src(c).  The
// permutation is chosen for the GEMM epilogues: an MFMA output lane owns one
// column of each 16-column block, so the columns are ordered so that one
// lane's blocks hold adjacent outputs:
//   Linear1 (N = 2I, rows interleaved gate/up by 8; c = 64G + 16b + j,
//     b = 0..3, j = 0..15): block b < 2 holds the gate row and block b + 2
//     the up row of channel 32G + 2j + (b & 1), so a lane holds both inputs
//     of two adjacent outputs (no cross-lane exchange before the SwiGLU) and
//     a 64-column group is one 32-channel requant group;
//   Linear2 (N = H; c = 128S + 16b + j, b = 0..7, j = 0..15): column
//     128S + 8j + b, so a lane that owns all eight blocks of a 128-column
//     span holds eight adjacent BF16 outputs (16 bytes), and one that owns
//     four of them (a 64-column wave tile) holds four (8 bytes).
//
// Linear2's activation scales use the analogous per-row-block layout
//   [R/BM][K/128][BM rows][4 B],
// written that way by the Linear1 epilogue.
#include "moe_internal.h"

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

// Weight row (within its 256-row block) stored at tile column c.
__device__ __forceinline__ int tile_source_col(int which, int c) {
    const int G = c >> 6, b = (c >> 4) & 3, j = c & 15;
    if (which == 1) {
        const int ch = G * 32 + j * 2 + (b & 1);           // SwiGLU channel within the block
        return (ch >> 3) * 16 + (ch & 7) + (b & 2) * 4;    // its gate (b < 2) or up row
    }
    const int S = c >> 7, b8 = (c >> 4) & 7;
    return S * 128 + j * 8 + b8;
}

__global__ __launch_bounds__(kThreads) void tile_weight_data_kernel(const uint8_t* __restrict__ w, int which, int N,
                                                                    int K, int64_t n_slots,
                                                                    uint8_t* __restrict__ out) {
    const int64_t s = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // output slot
    if (s >= n_slots) return;
    const int KT = K / 128, NT = N / 256;
    const int p = (int)(s & 1023);
    int64_t blk = s >> 10;                       // ((e * NT) + nt) * KT + kt
    const int kt = (int)(blk % KT);
    blk /= KT;
    const int nt = (int)(blk % NT);
    const int64_t e = blk / NT;
    const int c = p >> 2;
    const int q = (p & 3) ^ ((c >> 1) & 3);
    const int64_t col = (int64_t)nt * 256 + tile_source_col(which, c);
    const uint8_t* src = w + (e * N + col) * (K / 2) + (int64_t)kt * 64 + q * 16;
    *reinterpret_cast<v4i*>(out + s * 16) = *reinterpret_cast<const v4i*>(src);
}

__global__ __launch_bounds__(kThreads) void tile_weight_scale_kernel(const uint8_t* __restrict__ sf, int which, int N,
                                                                     int K, int64_t n_words,
                                                                     uint32_t* __restrict__ out) {
    const int64_t s = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // output word
    if (s >= n_words) return;
    const int KT = K / 128, NT = N / 256;
    const int c = (int)(s & 255);
    int64_t blk = s >> 8;
    const int kt = (int)(blk % KT);
    blk /= KT;
    const int nt = (int)(blk % NT);
    const int64_t e = blk / NT;
    const int64_t col = (int64_t)nt * 256 + tile_source_col(which, c);
    out[s] = *reinterpret_cast<const uint32_t*>(sf + (e * N + col) * (K / 32) + (int64_t)kt * 4);
}

}  // namespace

hipError_t launch_tile_weights(int which, int N, int K, int E, const uint8_t* w, const uint8_t* w_sf,
                               uint8_t* w_out, uint8_t* sf_out, hipStream_t stream) {
    const int64_t slots = (int64_t)E * N * K / 32;      // 16-byte slots = E*N*(K/2)/16
    const int64_t words = (int64_t)E * N * K / 128;
    if (slots > 0)
        hipLaunchKernelGGL(tile_weight_data_kernel, dim3((unsigned)((slots + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, stream, w, which, N, K, slots, w_out);
    if (words > 0)
        hipLaunchKernelGGL(tile_weight_scale_kernel, dim3((unsigned)((words + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, stream, w_sf, which, N, K, words,
                           reinterpret_cast<uint32_t*>(sf_out));
    return hipGetLastError();
}

}  // namespace moe
