// Tile forward, bf16 inputs, head_dim 128, for gfx950 (MI355X).
//
// One GPU's 2-D tile of the Q-KV matrix (Mesh-Attention tutorial page, "From
// 1-D ring to 2-D mesh"): for each Q slot, attention over the KV slots listed
// for it, FULL blocks entirely, DIAG blocks up to the diagonal, SKIP blocks
// not at all; the result is a partial output and log-sum-exp per query row.
//
// Work decomposition
//   workgroup = 4 waves sharing one KV head; each wave owns 32 query rows of
//               one query head (GQA: the waves of a workgroup are different
//               query heads of the same KV group when G > 1).
//   K/V are streamed through LDS in tiles of 64 keys, loaded once per
//   workgroup and read by all 4 waves.
//
// Matrix-core formulation (v_mfma_f32_32x32x16_bf16, 64-lane waves)
//   S^T = K Q^T: A = K tile (32 keys x 16 dims), B = Q^T (16 dims x 32 rows).
//     In the 32x32 accumulator, lane l holds query row l%32 and 16 keys,
//     key = 8*(i/4) + 4*(l/32) + i%4 for register i.  A query row thus lives
//     in one lane pair (l, l^32): row max/sum need one cross-half exchange
//     (v_permlane32_swap) per tile.
//   O^T += V^T P^T: A = V^T (32 dims x 16 keys), B = P^T straight from the
//     softmax registers (no shuffles).  The dot-product index of an MFMA only
//     has to be paired consistently between A and B, so B's keys follow the
//     accumulator order above and V^T is read in the same key order.
//
// LDS layouts (64-lane reads and writes free of bank conflicts)
//   K: row-major [64 keys][128 dims] bf16; the 16-byte chunk c of key row n
//      is stored at chunk c ^ (n & 15).
//   V: quad-interleaved: keys grouped in fours; for quad qd and dim d the 4
//      bf16 values (keys 4qd..4qd+3) form one 8-byte slot at index
//      qd*128 + (d ^ f(d, qd)), f = ((d >> 5) & 3) | ((qd & 1) << 2).  One
//      8-byte read gives the 4 consecutive keys an MFMA A-operand half needs.
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "tile_common.hpp"

namespace mesh_attn {
namespace {

using dev::kNegInf;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;      // head dim
constexpr int BN = 64;      // keys per LDS tile
constexpr int NW = kTileWaves;
constexpr int NT = NW * 64;
constexpr int kTileBytes = BN * D * 2;  // 16 KiB per K or V tile

static_assert(NT == 256, "the cooperative K/V loaders assume 256 threads");

__device__ __forceinline__ int v_slot(int qd, int d) {
    return qd * D + (d ^ (((d >> 5) & 3) | ((qd & 1) << 2)));
}

// Loads keys n0..n0+63 of one KV head into LDS (zero rows at or past L).
__device__ __forceinline__ void load_kv_tile(const __bf16* __restrict__ kslot,
                                             const __bf16* __restrict__ vslot, int n0, int L,
                                             size_t row_stride, unsigned char* sk,
                                             unsigned char* sv, int tid) {
    // K: 1024 chunks of 16 bytes, 4 per thread.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int ci = tid + NT * r;
        const int key = ci >> 4, ch = ci & 15;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (n0 + key < L)
            val = *reinterpret_cast<const u32x4*>(kslot + (size_t)(n0 + key) * row_stride + ch * 8);
        *reinterpret_cast<u32x4*>(sk + key * (D * 2) + ((ch ^ (key & 15)) << 4)) = val;
    }
    // V: thread owns dims 8*dg..8*dg+7 of keys 4*kq..4*kq+3.
    const int dg = tid & 15, kq = tid >> 4;
    u32x4 x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int key = 4 * kq + j;
        x[j] = u32x4{0u, 0u, 0u, 0u};
        if (n0 + key < L)
            x[j] = *reinterpret_cast<const u32x4*>(vslot + (size_t)(n0 + key) * row_stride + dg * 8);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        const bool hi = e & 1;
        u32x2 out;
        if (hi) {
            out[0] = (x[0][w] >> 16) | (x[1][w] & 0xffff0000u);
            out[1] = (x[2][w] >> 16) | (x[3][w] & 0xffff0000u);
        } else {
            out[0] = (x[0][w] & 0xffffu) | (x[1][w] << 16);
            out[1] = (x[2][w] & 0xffffu) | (x[3][w] << 16);
        }
        *reinterpret_cast<u32x2*>(sv + v_slot(kq, dg * 8 + e) * 8) = out;
    }
}

__global__ __launch_bounds__(NT, 2) void tile_fwd_bf16_d128(const TileParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kTileBytes];
    unsigned char* sk = smem;
    unsigned char* sv = smem + kTileBytes;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, r32 = lane & 31;
    const int L = p.part_len;
    const dev::WorkItem w = dev::decode_work(p, wave);
    const int u = w.wave_tok0 + r32;  // query offset in its partition
    const bool q_valid = u < L;
    const size_t q_row = (size_t)(w.q_slot * L + u) * p.heads_q + w.head;

    // Q^T fragments: for d-chunk c, lane holds q[u][h][16c + 8g .. 16c + 8g + 7].
    bf16x8 qf[8];
    {
        const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + q_row * D + 8 * g;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            u32x4 t = {0u, 0u, 0u, 0u};
            if (q_valid) t = *reinterpret_cast<const u32x4*>(qp + 16 * c);
            qf[c] = __builtin_bit_cast(bf16x8, t);
        }
    }

    f32x16 o_acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o_acc[t][i] = 0.0f;
    float m = kNegInf;  // running max of scaled base-2 scores
    float l = 0.0f;     // running exponent sum (this lane's keys)
    const float c2 = p.scale_log2e;
    const int wave_last_tok = min(L, w.wave_tok0 + 32) - 1;
    const size_t kv_row_stride = (size_t)p.heads_kv * D;

    const int b_end = p.sched.blk_off[w.q_slot + 1];
    for (int bi = p.sched.blk_off[w.q_slot]; bi < b_end; ++bi) {
        const int ent = p.sched.blk[bi];
        const int kv_slot = ent >> 2;
        const bool diag = (ent & 3) == kDiag;
        const int n_end = diag ? w.wg_tok_end : L;
        const __bf16* kslot = reinterpret_cast<const __bf16*>(p.k) +
                              ((size_t)kv_slot * L * p.heads_kv + w.kv_head) * D;
        const __bf16* vslot = reinterpret_cast<const __bf16*>(p.v) +
                              ((size_t)kv_slot * L * p.heads_kv + w.kv_head) * D;
        for (int n0 = 0; n0 < n_end; n0 += BN) {
            __syncthreads();
            load_kv_tile(kslot, vslot, n0, L, kv_row_stride, sk, sv, tid);
            __syncthreads();
            if (diag && n0 > wave_last_tok) continue;  // every key after every query

            // S^T = K Q^T for keys n0 .. n0+63 (two 32-key halves).
            f32x16 s[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int i = 0; i < 16; ++i) s[h][i] = 0.0f;
                const int key = 32 * h + r32;
                const unsigned char* krow = sk + key * (D * 2);
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int ch = (2 * c + g) ^ (key & 15);
                    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + (ch << 4));
                    s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[c], s[h], 0, 0, 0);
                }
            }

            // Causal diagonal and ragged tail: hide keys after the query or past L.
            if ((diag && n0 + BN - 1 > w.wave_tok0) || n0 + BN > L) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = n0 + 32 * h + 8 * (i >> 2) + 4 * g + (i & 3);
                        if (key >= L || (diag && key > u)) s[h][i] = kNegInf;
                    }
            }

            // Online softmax for this lane's row.
            float mx = kNegInf;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[h][i]);
            mx = dev::max_with_partner(mx);
            const float m_new = fmaxf(m, mx * c2);
            const float m_use = m_new == kNegInf ? 0.0f : m_new;
            const float alpha = dev::fast_exp2(m - m_use);
            m = m_new;
            l *= alpha;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) o_acc[t][i] *= alpha;

            bf16x8 pb[4];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float pv = dev::fast_exp2(__builtin_fmaf(s[h][i], c2, -m_use));
                    l += pv;
                    pb[2 * h + (i >> 3)][i & 7] = static_cast<__bf16>(pv);
                }

            // O^T += V^T P^T, 16 keys per MFMA.
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int qa = 4 * ks + g, qb = 4 * ks + 2 + g;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int d = 32 * t + r32;
                    const u32x2 va = *reinterpret_cast<const u32x2*>(sv + v_slot(qa, d) * 8);
                    const u32x2 vb = *reinterpret_cast<const u32x2*>(sv + v_slot(qb, d) * 8);
                    const u32x4 a4 = {va[0], va[1], vb[0], vb[1]};
                    o_acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, a4), pb[ks], o_acc[t], 0, 0, 0);
                }
            }
        }
    }

    // Epilogue: O = O_acc / l, lse = ln(2) * (m + log2 l); empty rows -> (0, -inf).
    const float l_tot = dev::add_with_partner(l);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (q_valid) {
        __bf16* op = reinterpret_cast<__bf16*>(p.o) + q_row * D;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                bf16x4 ov;
#pragma unroll
                for (int j = 0; j < 4; ++j) ov[j] = static_cast<__bf16>(o_acc[t][4 * ib + j] * inv);
                *reinterpret_cast<bf16x4*>(op + 32 * t + 8 * ib + 4 * g) = ov;
            }
        if (g == 0)
            p.lse[q_row] = l_tot > 0.0f ? (m + __log2f(l_tot)) * dev::kLn2 : kNegInf;
    }
}

}  // namespace

hipError_t launch_tile_fwd_bf16(const TileParams& p, int head_dim, hipStream_t stream) {
    if (head_dim != D) return hipErrorInvalidValue;
    const unsigned n_wg = static_cast<unsigned>(p.n_q_slots) * p.n_tok_blocks * p.heads_kv *
                          p.n_head_groups;
    hipLaunchKernelGGL(tile_fwd_bf16_d128, dim3(n_wg), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mesh_attn
