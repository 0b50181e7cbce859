// Row dot products D = sum_d dout * o for the attention backward (the term
// subtracted in dS = P (dP - D)), for gfx950.
//
// Bandwidth bound: every row is read once from each input.  A group of G
// lanes (G the power of two at or above the row's 16-byte chunk count, at
// most 64) owns one row; lane j reads chunks j, j+G, ... with 16-byte loads
// and the group reduces with cross-lane shuffles.  Consecutive groups own
// consecutive rows, so a wave reads a contiguous span.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace mesh_attn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dot_chunk(const u32x4 a, const u32x4 b, bool bf16) {
    if (!bf16) {
        const f32x4 x = __builtin_bit_cast(f32x4, a);
        const f32x4 y = __builtin_bit_cast(f32x4, b);
        return x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // bf16 -> f32 is a 16-bit shift of the bit pattern
        s += __uint_as_float(a[i] << 16) * __uint_as_float(b[i] << 16);
        s += __uint_as_float(a[i] & 0xffff0000u) * __uint_as_float(b[i] & 0xffff0000u);
    }
    return s;
}

template <bool BF16>
__global__ __launch_bounds__(256) void bwd_delta_kernel(int64_t rows, int chunks, int group_log2,
                                                        const u32x4* __restrict__ o,
                                                        const u32x4* __restrict__ dout,
                                                        float* __restrict__ delta) {
    const int G = 1 << group_log2;
    const int lane_in = threadIdx.x & (G - 1);
    const int64_t groups_per_block = blockDim.x >> group_log2;
    const int64_t first = static_cast<int64_t>(blockIdx.x) * groups_per_block +
                          (threadIdx.x >> group_log2);
    const int64_t stride = static_cast<int64_t>(gridDim.x) * groups_per_block;
    for (int64_t row = first; row < rows; row += stride) {
        float s = 0.0f;
        for (int c = lane_in; c < chunks; c += G) {
            const int64_t idx = row * chunks + c;
            s += dot_chunk(__builtin_nontemporal_load(o + idx), __builtin_nontemporal_load(dout + idx),
                           BF16);
        }
        for (int m = G >> 1; m > 0; m >>= 1) s += __shfl_xor(s, m, 64);
        if (lane_in == 0) delta[row] = s;
    }
}

}  // namespace

hipError_t launch_bwd_delta(int64_t rows, int head_dim, int dtype, const void* o, const void* dout,
                            float* delta, hipStream_t stream) {
    const bool bf16 = dtype == 0;
    const int chunks = head_dim / (bf16 ? 8 : 4);  // 16-byte chunks per row
    int g_log2 = 0;
    while ((1 << g_log2) < chunks && g_log2 < 6) ++g_log2;
    const int threads = 256;
    const int64_t rows_per_block = threads >> g_log2;
    const int64_t want = (rows + rows_per_block - 1) / rows_per_block;
    // one row group per thread group: a fully populated grid keeps the most loads in flight
    const unsigned grid = static_cast<unsigned>(want < (1 << 20) ? want : (1 << 20));
    const auto* op = static_cast<const u32x4*>(o);
    const auto* dp = static_cast<const u32x4*>(dout);
    if (bf16)
        hipLaunchKernelGGL(bwd_delta_kernel<true>, dim3(grid), dim3(threads), 0, stream, rows, chunks,
                           g_log2, op, dp, delta);
    else
        hipLaunchKernelGGL(bwd_delta_kernel<false>, dim3(grid), dim3(threads), 0, stream, rows,
                           chunks, g_log2, op, dp, delta);
    return hipGetLastError();
}

}  // namespace mesh_attn
