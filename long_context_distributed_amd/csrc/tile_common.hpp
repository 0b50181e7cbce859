// Device helpers shared by the tile-forward kernels: work-item decoding, the
// causal/ragged mask and the online-softmax state.
//
// Online softmax (ring-attention page, log-sum-exp section; FlashAttention is
// cited on the mlsanity page): each query row keeps a running maximum m and a
// running exponent sum l; when a new block of scores raises the maximum, the
// accumulated output and l are rescaled by exp(m_old - m_new).  Scores are
// kept in base 2: x2 = x * scale * log2(e), so exp(scale*x - m) becomes
// exp2(x2 - m2) and one v_exp_f32 per score suffices.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mesh_attn {
namespace dev {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.69314718055994530942f;

// Value of the same register in lane (l ^ 32), combined with op.
__device__ __forceinline__ float max_with_partner(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float add_with_partner(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// One workgroup's share of a tile.
struct WorkItem {
    int q_slot;
    int kv_head;
    int head;      // query head of this wave
    int wg_tok0;   // first token (partition offset) of the workgroup
    int wave_tok0; // first token of this wave's rows
    int wg_tok_end;  // one past the workgroup's last valid token (<= L)
};

// Workgroup index -> work item.  KV head varies fastest, then query-head
// group, then token block (highest first: in a DIAG block later tokens see
// more keys), then Q slot in heaviest-first order.  Works for every
// parameter struct with the forward's decomposition fields (TileParams,
// BwdDqParams); callable on the host so that the grid's coverage can be
// checked there.
template <typename Params>
__host__ __device__ inline WorkItem decode_work_at(const Params& p, int lam, int wave) {
    WorkItem w;
    w.kv_head = lam % p.heads_kv;
    lam /= p.heads_kv;
    const int hg = lam % p.n_head_groups;
    lam /= p.n_head_groups;
    const int tbi = lam % p.n_tok_blocks;
    const int rank = lam / p.n_tok_blocks;
    w.q_slot = p.sched.q_order[rank];
    const int tb = p.n_tok_blocks - 1 - tbi;
    const int h_in = wave % p.heads_per_wg;
    const int tg = wave / p.heads_per_wg;
    w.head = w.kv_head * p.group + hg * p.heads_per_wg + h_in;
    w.wg_tok0 = tb * p.wave_rows * p.tok_groups;
    w.wave_tok0 = w.wg_tok0 + p.wave_rows * tg;
    const int wg_end = w.wg_tok0 + p.wave_rows * p.tok_groups;
    w.wg_tok_end = wg_end < p.part_len ? wg_end : p.part_len;
    return w;
}

template <typename Params>
__device__ __forceinline__ WorkItem decode_work(const Params& p, int wave) {
    return decode_work_at(p, static_cast<int>(blockIdx.x), wave);
}

// Workgroup index of the key/value-gradient kernel -> (KV slot, key block,
// KV head); the KV head varies fastest.
struct KeyBlock {
    int kv_slot;
    int key_block;
    int kv_head;
};

template <typename Params>
__host__ __device__ inline KeyBlock decode_key_block_at(const Params& p, int lam) {
    KeyBlock b;
    b.kv_head = lam % p.heads_kv;
    lam /= p.heads_kv;
    b.key_block = lam % p.n_key_blocks;
    b.kv_slot = lam / p.n_key_blocks;
    return b;
}

}  // namespace dev
}  // namespace mesh_attn
