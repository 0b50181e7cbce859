// Internal interface between the C-ABI layer (api.cpp) and the HIP kernels.
// Not installed; the public interface is include/mesh_attn.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "mesh_attn.h"

namespace mesh_attn {

constexpr int kMaxQSlots = 64;
constexpr int kMaxKvSlots = 64;
constexpr int kMaxBlocks = 1024;

// Block classes as stored in the packed schedule (same values as the ABI).
constexpr int kFull = 0;
constexpr int kDiag = 1;
constexpr int kSkip = 2;

// Which KV slots each Q slot attends to, packed into the kernel arguments.
// For Q slot s the entries blk[blk_off[s] .. blk_off[s+1]) are
// (kv_slot << 2) | kind, non-SKIP blocks only, in KV-slot (rotation) order.
// q_order lists Q slots heaviest first (FULL = 1, DIAG = 1/2) so that the
// longest work items are dispatched first.
struct TileSchedule {
    uint8_t blk[kMaxBlocks];  // first, so that it is 4-byte aligned (read as dwords)
    uint8_t q_order[kMaxQSlots];
    uint16_t blk_off[kMaxQSlots + 2];  // one spare entry keeps the size a multiple of 4
};

// Entry i of the packed schedule, read as a dword so that a wave-uniform
// index becomes a scalar load (there are no scalar byte loads on gfx9).
__host__ __device__ __forceinline__ int sched_entry(const TileSchedule& s, int i) {
    const uint32_t word = reinterpret_cast<const uint32_t*>(s.blk)[i >> 2];
    return (word >> (8 * (i & 3))) & 0xff;
}

static_assert(sizeof(TileSchedule) % 4 == 0, "schedule size");

// Arguments of one tile-forward launch.  The grid is a flat list of work
// items (Q slot rank, token block, KV head, query-head group); KV head varies
// fastest so that work items sharing K/V land on the same XCD.
struct TileParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int32_t part_len;      // L
    int32_t heads_q;       // H_q
    int32_t heads_kv;      // H_kv
    int32_t group;         // G = H_q / H_kv
    int32_t heads_per_wg;  // query heads of one KV group handled by a workgroup
    int32_t tok_groups;    // token row groups per workgroup (waves / heads_per_wg)
    int32_t wave_rows;     // query rows (tokens) per wave
    int32_t n_tok_blocks;  // ceil(L / (wave_rows * tok_groups))
    int32_t n_head_groups; // G / heads_per_wg
    int32_t n_q_slots;
    float scale_log2e;     // softmax_scale * log2(e)
    TileSchedule sched;
};

static_assert(offsetof(TileParams, sched) % 4 == 0, "schedule must be dword aligned");

// Waves per workgroup and query rows per wave of the tile kernels.  In the
// float32 kernel all waves of a workgroup share one block of rows and split
// its keys among themselves: kTileWavesF32 waves own rows (one), and
// kTileKeySplitF32 waves run per workgroup.
constexpr int kTileWavesBf16 = 12;
constexpr int kTileWavesF32 = 1;
constexpr int kTileKeySplitF32 = 4;
constexpr int kWaveRowsBf16 = 32;
constexpr int kWaveRowsF32 = 16;

// The same blocks seen from the KV side, for the key/value-gradient kernel:
// for KV slot j the entries blk[blk_off[j] .. blk_off[j+1]) are
// (q_slot << 2) | kind, non-SKIP blocks only, in Q-slot order.
struct KvSchedule {
    uint8_t blk[kMaxBlocks];
    uint16_t blk_off[kMaxKvSlots + 2];
};

static_assert(sizeof(KvSchedule) % 4 == 0, "schedule size");

// Arguments of the query-gradient kernel: Q-stationary, with the same work
// decomposition (and fields) as the forward.
struct BwdDqParams {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* lse;
    const float* delta;
    float* dq;
    int32_t part_len;
    int32_t heads_q;
    int32_t heads_kv;
    int32_t group;
    int32_t heads_per_wg;
    int32_t tok_groups;
    int32_t wave_rows;
    int32_t n_tok_blocks;
    int32_t n_head_groups;
    int32_t n_q_slots;
    float scale;           // softmax_scale
    float scale_log2e;     // softmax_scale * log2(e)
    TileSchedule sched;
};

static_assert(offsetof(BwdDqParams, sched) % 4 == 0, "schedule must be dword aligned");

// Arguments of the key/value-gradient kernel: KV-stationary.  The grid is
// (KV slot, key block, KV head) with the KV head varying fastest.
struct BwdDkvParams {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* lse;
    const float* delta;
    float* dk;
    float* dv;
    int32_t part_len;
    int32_t heads_q;
    int32_t heads_kv;
    int32_t group;
    int32_t n_kv_slots;
    int32_t n_key_blocks;  // ceil(L / keys per workgroup)
    float scale;
    float scale_log2e;
    KvSchedule sched;
};

static_assert(offsetof(BwdDkvParams, sched) % 4 == 0, "schedule must be dword aligned");

// Waves per workgroup of the backward kernels; every wave owns 32 query rows
// (query-gradient kernel) or 32 keys (key/value-gradient kernel).
constexpr int kBwdDqWaves = 8;
constexpr int kBwdDkvWaves = 8;
constexpr int kBwdRowsPerWave = 32;

// Workgroups of a forward-decomposed launch (tile forward, query-gradient
// kernel) and of the key/value-gradient kernel.
template <typename Params>
inline int64_t tile_fwd_grid(const Params& p) {
    return static_cast<int64_t>(p.n_q_slots) * p.n_tok_blocks * p.heads_kv * p.n_head_groups;
}
inline int64_t tile_bwd_dkdv_grid(const BwdDkvParams& p) {
    return static_cast<int64_t>(p.n_kv_slots) * p.n_key_blocks * p.heads_kv;
}

// Host planning of a tile call: validates the description, packs the
// schedule and sets the work decomposition (tensor pointers are left NULL).
// Returns a status; the entry points launch what these produce.
int plan_tile_fwd(const char* who, const mesh_attn_tile_desc& d, TileParams& p);
int plan_tile_bwd(const char* who, const mesh_attn_tile_desc& d, BwdDqParams& pq, BwdDkvParams& pk);

hipError_t launch_tile_fwd_bf16(const TileParams& p, int head_dim, hipStream_t stream);
hipError_t launch_tile_fwd_f32(const TileParams& p, int head_dim, hipStream_t stream);

hipError_t launch_tile_bwd_bf16(const BwdDqParams& pq, const BwdDkvParams& pk, int head_dim,
                               hipStream_t stream);
hipError_t launch_bwd_delta(int64_t rows, int head_dim, int dtype, const void* o, const void* dout,
                            float* delta, hipStream_t stream);

hipError_t launch_lse_merge(int n_parts, int64_t rows, int head_dim, int dtype,
                            const void* o_parts, const float* lse_parts, void* o_out,
                            float* lse_out, hipStream_t stream);

}  // namespace mesh_attn
