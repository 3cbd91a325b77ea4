// Top-k combine: y[t] = BF16( sum over j ascending of float(Yslot[slot[t, j]]) )
// with the sum in FP32 and tokens without a local hit written as +0
// (walk-through section 4.6 "combine reduction"; reading notes "stage six").
// The routing weight was applied in the Linear1 epilogue, so the sum is
// unweighted.  If the forward's status word reports that a single-launch GEMM gave up waiting for
// its Linear1 rows (so some slot rows may be wrong), every element of y is written as NaN instead.
//
// HBM-bound: each thread owns 8 consecutive BF16 columns of one token at a time (one 16-byte load per
// slot), a workgroup 256 such spans of one token (blockIdx.x = token, blockIdx.y = first span block),
// so a wave reads whole 1 KiB spans of each slot row.  A thread issues the loads of up to 8 slots
// before it adds any of them (in j order), so one memory round trip covers them.  Small batches spread
// each token over several workgroups to fill the GPU; large ones keep the grid near kMaxBlocks
// workgroups and loop over the span blocks.
#include "moe_internal.h"

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kBatch = 8;  // slot loads in flight per thread
constexpr int kMaxBlocks = 32768;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

constexpr uint32_t kNaNPair = 0x7FC07FC0u;  // two BF16 quiet NaNs

__global__ __launch_bounds__(kThreads) void combine_kernel(const uint16_t* __restrict__ yslot,
                                                           const int32_t* __restrict__ slot, int k, int H,
                                                           const uint32_t* __restrict__ status,
                                                           uint16_t* __restrict__ y) {
    const int t = blockIdx.x;
    const int32_t* s = slot + (size_t)t * k;
    if (__builtin_amdgcn_readfirstlane(*status) != 0u) {
        const v4i nan = v4i{(int)kNaNPair, (int)kNaNPair, (int)kNaNPair, (int)kNaNPair};
        for (int c = blockIdx.y * kThreads + threadIdx.x; c < H / 8; c += gridDim.y * kThreads)
            *reinterpret_cast<v4i*>(y + (size_t)t * H + c * 8) = nan;
        return;
    }
    for (int c = blockIdx.y * kThreads + threadIdx.x; c < H / 8; c += gridDim.y * kThreads) {  // 8-column span
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0; j0 < k; j0 += kBatch) {
            v4i v[kBatch];
            bool ok[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int r = j0 + u < k ? s[j0 + u] : -1;
                ok[u] = r >= 0;
                // slot rows are read exactly once: non-temporal, so they do not evict other lines
                v[u] = ok[u] ? __builtin_nontemporal_load(reinterpret_cast<const v4i*>(yslot + (size_t)r * H + c * 8))
                             : v4i{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (!ok[u]) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] += bf16_lo((uint32_t)v[u][q]);
                    acc[2 * q + 1] += bf16_hi((uint32_t)v[u][q]);
                }
            }
        }
        v4i out;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)acc[2 * q]);
            const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)acc[2 * q + 1]);
            out[q] = (int)(lo | (hi << 16));
        }
        __builtin_nontemporal_store(out, reinterpret_cast<v4i*>(y + (size_t)t * H + c * 8));
    }
}

}  // namespace

hipError_t launch_combine(const moe_shape& s, const uint16_t* yslot, const int32_t* slot, const uint32_t* status,
                          uint16_t* y, hipStream_t stream) {
    if (s.num_tokens == 0) return hipSuccess;
    const int blocks = (s.hidden / 8 + kThreads - 1) / kThreads;  // span blocks per token
    const dim3 grid((unsigned)s.num_tokens, (unsigned)std::max(1, std::min(blocks, kMaxBlocks / s.num_tokens)));
    hipLaunchKernelGGL(combine_kernel, grid, dim3(kThreads), 0, stream, yslot, slot, s.topk, s.hidden, status, y);
    return hipGetLastError();
}

}  // namespace moe
