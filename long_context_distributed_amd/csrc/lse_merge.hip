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
// The loads of all partials of a chunk are issued before any is used (the
// partial count is a template bound), and the once-read partials and the
// output use non-temporal accesses so they do not displace other data in
// the caches.
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

// Two 16-byte chunks of one output row per thread and grid-stride step
// (rows hold an even number of chunks).  NMAX bounds the number of
// partials so that all their loads are unrolled and in flight together;
// partials past n are masked off.
template <bool BF16, int NMAX>
__global__ __launch_bounds__(NT) void lse_merge_kernel(int n, int64_t rows, int chunks_per_row,
                                                       const u32x4* __restrict__ o_parts,
                                                       const float* __restrict__ lse_parts,
                                                       u32x4* __restrict__ o_out,
                                                       float* __restrict__ lse_out) {
    using C = Chunk<BF16>;
    const int64_t total = rows * chunks_per_row;
    const int half = chunks_per_row / 2;
    const int64_t pairs = total / 2;
    for (int64_t pidx = (int64_t)blockIdx.x * NT + threadIdx.x; pidx < pairs;
         pidx += (int64_t)gridDim.x * NT) {
        // Chunks c and c + C/2 of one row: consecutive lanes then cover whole
        // row segments, so every load and store instruction is contiguous.
        const int64_t row = pidx / half;
        const int ch = static_cast<int>(pidx - row * half);
        const int64_t idx = row * chunks_per_row + ch;
        const int64_t idx1 = idx + half;
        float li[NMAX];
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < NMAX; ++i) {
            li[i] = i < n ? lse_parts[(int64_t)i * rows + row] : kNegInf;
            mx = fmaxf(mx, li[i]);
        }
        float acc0[C::N], acc1[C::N];
#pragma unroll
        for (int j = 0; j < C::N; ++j) {
            acc0[j] = 0.0f;
            acc1[j] = 0.0f;
        }
        float wsum = 0.0f;
        if (mx != kNegInf) {
            u32x4 r0[NMAX], r1[NMAX];
            float w[NMAX];
#pragma unroll
            for (int i = 0; i < NMAX; ++i) {
                w[i] = __builtin_amdgcn_exp2f((li[i] - mx) * kLog2e);
                r0[i] = u32x4{0u, 0u, 0u, 0u};
                r1[i] = r0[i];
                if (li[i] != kNegInf) {  // dead partials are not read
                    r0[i] = __builtin_nontemporal_load(&o_parts[(int64_t)i * total + idx]);
                    r1[i] = __builtin_nontemporal_load(&o_parts[(int64_t)i * total + idx1]);
                }
            }
#pragma unroll
            for (int i = 0; i < NMAX; ++i) {
                wsum += w[i];
                if (w[i] != 0.0f) {
                    C::add(acc0, w[i], r0[i]);
                    C::add(acc1, w[i], r1[i]);
                }
            }
        }
        const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
        __builtin_nontemporal_store(C::pack(acc0, inv), &o_out[idx]);
        __builtin_nontemporal_store(C::pack(acc1, inv), &o_out[idx1]);
        if (lse_out != nullptr && ch == 0)
            lse_out[row] = wsum > 0.0f ? mx + __log2f(wsum) * kLn2 : kNegInf;
    }
}

// Any number of partials and any chunk count: one chunk per thread and
// step, partials in groups of eight (same arithmetic).
template <bool BF16>
__global__ __launch_bounds__(NT) void lse_merge_kernel_any(int n, int64_t rows, int chunks_per_row,
                                                           const u32x4* __restrict__ o_parts,
                                                           const float* __restrict__ lse_parts,
                                                           u32x4* __restrict__ o_out,
                                                           float* __restrict__ lse_out) {
    using C = Chunk<BF16>;
    const int64_t total = rows * chunks_per_row;
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
            for (int i0 = 0; i0 < n; i0 += 8) {
                float w[8];
                u32x4 raw[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int i = i0 + t;
                    w[t] = 0.0f;
                    raw[t] = u32x4{0u, 0u, 0u, 0u};
                    if (i < n) {
                        const float li = lse_parts[(int64_t)i * rows + row];
                        w[t] = __builtin_amdgcn_exp2f((li - mx) * kLog2e);
                        if (li != kNegInf) raw[t] = __builtin_nontemporal_load(&o_parts[(int64_t)i * total + idx]);
                    }
                }
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    wsum += w[t];
                    if (w[t] != 0.0f) C::add(acc, w[t], raw[t]);
                }
            }
        }
        const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
        __builtin_nontemporal_store(C::pack(acc, inv), &o_out[idx]);
        if (lse_out != nullptr && ch == 0)
            lse_out[row] = wsum > 0.0f ? mx + __log2f(wsum) * kLn2 : kNegInf;
    }
}

template <bool BF16>
hipError_t launch_typed(int n, int64_t rows, int chunks_per_row, const u32x4* o_parts,
                        const float* lse_parts, u32x4* o_out, float* lse_out, hipStream_t stream) {
    const int64_t total = rows * chunks_per_row;
    const bool pairs = chunks_per_row % 2 == 0 && n <= 16;
    // One work item per thread (a grid stride only past 2^20 workgroups): a
    // fully populated grid keeps more loads in flight than a smaller grid
    // that loops (measured on the 8 x 4Mi-row merge: 5.7 TB/s against 5.2
    // with 16384 workgroups).
    const int64_t want = ((pairs ? total / 2 : total) + NT - 1) / NT;
    const unsigned grid = static_cast<unsigned>(want < (1 << 20) ? want : (1 << 20));
#define MESH_ATTN_MERGE(NMAX)                                                                      \
    hipLaunchKernelGGL((lse_merge_kernel<BF16, NMAX>), dim3(grid), dim3(NT), 0, stream, n, rows,   \
                       chunks_per_row, o_parts, lse_parts, o_out, lse_out)
    if (!pairs)
        hipLaunchKernelGGL(lse_merge_kernel_any<BF16>, dim3(grid), dim3(NT), 0, stream, n, rows,
                           chunks_per_row, o_parts, lse_parts, o_out, lse_out);
    else if (n <= 2)
        MESH_ATTN_MERGE(2);
    else if (n <= 4)
        MESH_ATTN_MERGE(4);
    else if (n <= 8)
        MESH_ATTN_MERGE(8);
    else
        MESH_ATTN_MERGE(16);
#undef MESH_ATTN_MERGE
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(int n_parts, int64_t rows, int head_dim, int dtype,
                            const void* o_parts, const float* lse_parts, void* o_out,
                            float* lse_out, hipStream_t stream) {
    const bool bf16 = dtype == 0;
    const int chunks_per_row = head_dim / (bf16 ? 8 : 4);
    const u32x4* src = static_cast<const u32x4*>(o_parts);
    u32x4* dst = static_cast<u32x4*>(o_out);
    return bf16 ? launch_typed<true>(n_parts, rows, chunks_per_row, src, lse_parts, dst, lse_out, stream)
                : launch_typed<false>(n_parts, rows, chunks_per_row, src, lse_parts, dst, lse_out, stream);
}

}  // namespace mesh_attn
