// LSE merge of partial attention results, for gfx950 (MI355X).
//
// The owner of a Q partition receives partial outputs from its mesh-row peers
// (Mesh-Attention tutorial page, greedy-algorithm section) and combines them
// with log-sum-exp weights (ring-attention page, log-sum-exp section; its
// printed decomposition omits the weights): per row,
//   M = max_i lse_i,  w_i = exp(lse_i - M),
//   o = sum_i w_i o_i / sum_i w_i,  lse = M + ln(sum_i w_i),
// and a row whose partials are all -inf becomes (0, -inf).
//
// The kernel streams HBM: every thread owns one 16-byte chunk of one output
// row (8 bf16 or 4 f32 values), reads that chunk from each live partial and
// accumulates in float32.  Partials with lse = -inf are not read at all.
// Loads of four partials are issued before any of them is used, to keep
// enough bytes in flight.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mesh_attn {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int NT = 256;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994530942f;

template <bool BF16>
struct Chunk;

template <>
struct Chunk<true> {  // 8 bf16 values
    static constexpr int N = 8;
    __device__ static void add(float* acc, float w, u32x4 raw) {
        const bf16x8 x = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_fmaf(w, static_cast<float>(x[j]), acc[j]);
    }
    __device__ static u32x4 pack(const float* acc, float s) {
        bf16x8 x;
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = static_cast<__bf16>(acc[j] * s);
        return __builtin_bit_cast(u32x4, x);
    }
};

template <>
struct Chunk<false> {  // 4 float values
    static constexpr int N = 4;
    __device__ static void add(float* acc, float w, u32x4 raw) {
        const f32x4 x = __builtin_bit_cast(f32x4, raw);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_fmaf(w, x[j], acc[j]);
    }
    __device__ static u32x4 pack(const float* acc, float s) {
        f32x4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = acc[j] * s;
        return __builtin_bit_cast(u32x4, x);
    }
};

template <bool BF16>
__global__ __launch_bounds__(NT) void lse_merge_kernel(int n, int64_t rows, int chunks_per_row,
                                                       const u32x4* __restrict__ o_parts,
                                                       const float* __restrict__ lse_parts,
                                                       u32x4* __restrict__ o_out,
                                                       float* __restrict__ lse_out) {
    using C = Chunk<BF16>;
    const int64_t total = rows * chunks_per_row;
    const int64_t part_stride = total;  // chunks per partial
    for (int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * NT) {
        const int64_t row = idx / chunks_per_row;
        const int ch = static_cast<int>(idx - row * chunks_per_row);

        float mx = kNegInf;
        for (int i = 0; i < n; ++i) mx = fmaxf(mx, lse_parts[(int64_t)i * rows + row]);

        float acc[C::N];
#pragma unroll
        for (int j = 0; j < C::N; ++j) acc[j] = 0.0f;
        float wsum = 0.0f;
        if (mx != kNegInf) {
            for (int i0 = 0; i0 < n; i0 += 4) {
                float w[4];
                u32x4 raw[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int i = i0 + t;
                    w[t] = 0.0f;
                    raw[t] = u32x4{0u, 0u, 0u, 0u};
                    if (i < n) {
                        const float li = lse_parts[(int64_t)i * rows + row];
                        w[t] = __builtin_amdgcn_exp2f((li - mx) * kLog2e);
                        if (li != kNegInf) raw[t] = o_parts[(int64_t)i * part_stride + idx];
                    }
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    wsum += w[t];
                    if (w[t] != 0.0f) C::add(acc, w[t], raw[t]);
                }
            }
        }
        const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
        o_out[idx] = C::pack(acc, inv);
        if (lse_out != nullptr && ch == 0)
            lse_out[row] = wsum > 0.0f ? mx + __log2f(wsum) * kLn2 : kNegInf;
    }
}

}  // namespace

hipError_t launch_lse_merge(int n_parts, int64_t rows, int head_dim, int dtype,
                            const void* o_parts, const float* lse_parts, void* o_out,
                            float* lse_out, hipStream_t stream) {
    const bool bf16 = dtype == 0;
    const int chunks_per_row = head_dim / (bf16 ? 8 : 4);
    const int64_t total = rows * chunks_per_row;
    // Enough workgroups to fill the chip several times over; each thread then
    // loops over chunks with a grid stride.
    const int64_t want = (total + NT - 1) / NT;
    const unsigned grid = static_cast<unsigned>(want < 256 * 64 ? want : 256 * 64);
    if (bf16)
        hipLaunchKernelGGL(lse_merge_kernel<true>, dim3(grid), dim3(NT), 0, stream, n_parts, rows,
                           chunks_per_row, static_cast<const u32x4*>(o_parts), lse_parts,
                           static_cast<u32x4*>(o_out), lse_out);
    else
        hipLaunchKernelGGL(lse_merge_kernel<false>, dim3(grid), dim3(NT), 0, stream, n_parts, rows,
                           chunks_per_row, static_cast<const u32x4*>(o_parts), lse_parts,
                           static_cast<u32x4*>(o_out), lse_out);
    return hipGetLastError();
}

}  // namespace mesh_attn
