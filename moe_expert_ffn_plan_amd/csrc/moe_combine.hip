// Top-k combine: y[t] = BF16( sum over j ascending of float(Yslot[slot[t, j]]) )
// with the sum in FP32 and tokens without a local hit written as +0
// (walk-through section 4.6 "combine reduction"; reading notes "stage six").
// The routing weight was applied in the Linear1 epilogue, so the sum is
// unweighted.
//
// HBM-bound: one workgroup per token, each thread owning 8 consecutive BF16
// columns (one 16-byte load per slot), so a wave reads whole 1 KiB spans of
// each slot row and all k loads of a thread are in flight together.
#include "moe_internal.h"

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__global__ __launch_bounds__(kThreads) void combine_kernel(const uint16_t* __restrict__ yslot,
                                                           const int32_t* __restrict__ slot, int k, int H,
                                                           uint16_t* __restrict__ y) {
    const int t = blockIdx.x;
    const int32_t* s = slot + (size_t)t * k;
    for (int c = threadIdx.x; c < H / 8; c += kThreads) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; ++j) {
            const int r = s[j];
            if (r < 0) continue;
            const v4i v = *reinterpret_cast<const v4i*>(yslot + (size_t)r * H + c * 8);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += bf16_lo((uint32_t)v[q]);
                acc[2 * q + 1] += bf16_hi((uint32_t)v[q]);
            }
        }
        v4i out;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)acc[2 * q]);
            const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)acc[2 * q + 1]);
            out[q] = (int)(lo | (hi << 16));
        }
        *reinterpret_cast<v4i*>(y + (size_t)t * H + c * 8) = out;
    }
}

}  // namespace

hipError_t launch_combine(const moe_shape& s, const uint16_t* yslot, const int32_t* slot, uint16_t* y,
                          hipStream_t stream) {
    if (s.num_tokens == 0) return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3(s.num_tokens), dim3(kThreads), 0, stream, yslot, slot, s.topk,
                       s.hidden, y);
    return hipGetLastError();
}

}  // namespace moe
