// Tile forward, float32 inputs (head_dim 64 or 128), for gfx950 (MI355X).
//
// Same tile semantics as the bf16 kernel (Mesh-Attention tutorial page, "From
// 1-D ring to 2-D mesh"; online softmax as in the ring-attention page's
// log-sum-exp section) with float32 matrix-core math:
// v_mfma_f32_32x32x2_f32.  Each MFMA contracts over 2 elements, one per lane
// half, so both operands are single floats per lane:
//   S^T = K Q^T: A = K[key = l%32][d], B = Q[row = l%32][d]; the pair of
//     dims used by MFMA number c is d(c, half) = 8*(c/4) + 4*half + c%4, so
//     each lane reads 4 consecutive dims with one 16-byte load.
//   O^T += V^T P^T: MFMA number i contracts the two keys a lane pair holds in
//     accumulator register i (keys 8*(i/4) + 4*half + i%4); B is the softmax
//     value in that register, A is V[that key][d = l%32].
// LDS rows are padded (K by 4 floats, V by 8) so that the 64-lane reads hit
// distinct banks.
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "tile_common.hpp"

namespace mesh_attn {
namespace {

using dev::kNegInf;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BN = 32;  // keys per LDS tile
constexpr int NW = kTileWavesF32;
constexpr int NT = NW * 64;

template <int D>
__global__ __launch_bounds__(NT, 2) void tile_fwd_f32_kernel(const TileParams p) {
    constexpr int KS = D + 4;  // padded row strides (floats)
    constexpr int VS = D + 8;
    constexpr int DT = D / 32;  // output tiles of 32 dims
    __shared__ __attribute__((aligned(16))) float sk[BN * KS];
    __shared__ __attribute__((aligned(16))) float sv[BN * VS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, r32 = lane & 31;
    const int L = p.part_len;
    const dev::WorkItem w = dev::decode_work(p, wave);
    const int u = w.wave_tok0 + r32;
    const bool q_valid = u < L;
    const size_t q_row = (size_t)(w.q_slot * L + u) * p.heads_q + w.head;

    f32x4 qv[D / 8];
    {
        const float* qp = reinterpret_cast<const float*>(p.q) + q_row * D + 4 * g;
#pragma unroll
        for (int j = 0; j < D / 8; ++j) {
            qv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (q_valid) qv[j] = *reinterpret_cast<const f32x4*>(qp + 8 * j);
        }
    }

    f32x16 o_acc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o_acc[t][i] = 0.0f;
    float m = kNegInf, l = 0.0f;
    const float c2 = p.scale_log2e;
    const int wave_last_tok = min(L, w.wave_tok0 + 32) - 1;
    const size_t row_stride = (size_t)p.heads_kv * D;

    const int b_end = p.sched.blk_off[w.q_slot + 1];
    for (int bi = p.sched.blk_off[w.q_slot]; bi < b_end; ++bi) {
        const int ent = sched_entry(p.sched, bi);
        const int kv_slot = ent >> 2;
        const bool diag = (ent & 3) == kDiag;
        const int n_end = diag ? w.wg_tok_end : L;
        const float* kslot = reinterpret_cast<const float*>(p.k) +
                             ((size_t)kv_slot * L * p.heads_kv + w.kv_head) * D;
        const float* vslot = reinterpret_cast<const float*>(p.v) +
                             ((size_t)kv_slot * L * p.heads_kv + w.kv_head) * D;
        for (int n0 = 0; n0 < n_end; n0 += BN) {
            __syncthreads();
            constexpr int CPR = D / 4;  // 16-byte chunks per row
#pragma unroll
            for (int r = 0; r < BN * CPR / NT; ++r) {
                const int ci = tid + NT * r;
                const int key = ci / CPR, ch = ci % CPR;
                f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
                if (n0 + key < L) {
                    kx = *reinterpret_cast<const f32x4*>(kslot + (size_t)(n0 + key) * row_stride + 4 * ch);
                    vx = *reinterpret_cast<const f32x4*>(vslot + (size_t)(n0 + key) * row_stride + 4 * ch);
                }
                *reinterpret_cast<f32x4*>(sk + key * KS + 4 * ch) = kx;
                *reinterpret_cast<f32x4*>(sv + key * VS + 4 * ch) = vx;
            }
            __syncthreads();
            if (diag && n0 > wave_last_tok) continue;

            f32x16 s;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = 0.0f;
            const float* krow = sk + r32 * KS + 4 * g;
#pragma unroll
            for (int j = 0; j < D / 8; ++j) {
                const f32x4 ka = *reinterpret_cast<const f32x4*>(krow + 8 * j);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[e], qv[j][e], s, 0, 0, 0);
            }

            if ((diag && n0 + BN - 1 > w.wave_tok0) || n0 + BN > L) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = n0 + 8 * (i >> 2) + 4 * g + (i & 3);
                    if (key >= L || (diag && key > u)) s[i] = kNegInf;
                }
            }

            float mx = kNegInf;
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
            mx = dev::max_with_partner(mx);
            const float m_new = fmaxf(m, mx * c2);
            const float m_use = m_new == kNegInf ? 0.0f : m_new;
            const float alpha = dev::fast_exp2(m - m_use);
            m = m_new;
            l *= alpha;
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) o_acc[t][i] *= alpha;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s[i] = dev::fast_exp2(__builtin_fmaf(s[i], c2, -m_use));
                l += s[i];
            }

#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = 8 * (i >> 2) + 4 * g + (i & 3);
#pragma unroll
                for (int t = 0; t < DT; ++t)
                    o_acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(sv[key * VS + 32 * t + r32], s[i],
                                                                    o_acc[t], 0, 0, 0);
            }
        }
    }

    const float l_tot = dev::add_with_partner(l);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (q_valid) {
        float* op = reinterpret_cast<float*>(p.o) + q_row * D;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                f32x4 ov;
#pragma unroll
                for (int j = 0; j < 4; ++j) ov[j] = o_acc[t][4 * ib + j] * inv;
                *reinterpret_cast<f32x4*>(op + 32 * t + 8 * ib + 4 * g) = ov;
            }
        if (g == 0)
            p.lse[q_row] = l_tot > 0.0f ? (m + __log2f(l_tot)) * dev::kLn2 : kNegInf;
    }
}

}  // namespace

hipError_t launch_tile_fwd_f32(const TileParams& p, int head_dim, hipStream_t stream) {
    const unsigned n_wg = static_cast<unsigned>(tile_fwd_grid(p));
    if (head_dim == 64)
        hipLaunchKernelGGL(tile_fwd_f32_kernel<64>, dim3(n_wg), dim3(NT), 0, stream, p);
    else if (head_dim == 128)
        hipLaunchKernelGGL(tile_fwd_f32_kernel<128>, dim3(n_wg), dim3(NT), 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace mesh_attn
