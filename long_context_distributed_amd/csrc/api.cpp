// C-ABI entry points: host-side validation, packing of the tile schedule into
// kernel arguments, and launches on the caller's stream.
//
// Every argument is checked before the first HIP call, so every error path
// can be exercised on a machine without a GPU.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "mesh_attn.h"
#include "kernels.h"
#include "status.h"

namespace mesh_attn {

namespace {
thread_local std::string g_last_error;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) {
        clear_error();
        return MESH_ATTN_OK;
    }
    g_last_error = std::string(what) + ": " + hipGetErrorString(e);
    return MESH_ATTN_ERR_HIP;
}

int gcd(int a, int b) {
    while (b != 0) {
        const int t = a % b;
        a = b;
        b = t;
    }
    return a;
}
}  // namespace

int fail(int status, const char* msg) {
    g_last_error = msg;
    return status;
}

// "who: msg"
static int failw(int status, const char* who, const char* msg) {
    g_last_error = std::string(who) + ": " + msg;
    return status;
}

void clear_error() { g_last_error.clear(); }

// Checks a tile description's block list and packs it: Q-slot major into
// `qs` (with the heaviest-first Q-slot order) and, if `ks` is not NULL,
// KV-slot major into `ks`.  Returns a status.
static int build_schedule(const char* who, const mesh_attn_tile_desc& d, TileSchedule& qs,
                          KvSchedule* ks) {
    const int nq = d.n_q_slots, nkv = d.n_kv_slots;
    if (d.n_blocks < 0 || d.n_blocks > MESH_ATTN_MAX_BLOCKS)
        return failw(MESH_ATTN_ERR_INVALID, who, "n_blocks out of range");
    if (d.n_blocks > 0 && d.blocks == nullptr)
        return failw(MESH_ATTN_ERR_INVALID, who, "blocks is NULL");

    // kind of each (q_slot, kv_slot); -1 = not listed
    int8_t kind[kMaxQSlots][kMaxKvSlots];
    memset(kind, -1, sizeof(kind));
    int32_t q_part_of[kMaxQSlots], kv_part_of[kMaxKvSlots];
    for (int i = 0; i < kMaxQSlots; ++i) q_part_of[i] = -1;
    for (int i = 0; i < kMaxKvSlots; ++i) kv_part_of[i] = -1;

    for (int i = 0; i < d.n_blocks; ++i) {
        const mesh_attn_block& b = d.blocks[i];
        if (b.q_slot < 0 || b.q_slot >= nq || b.kv_slot < 0 || b.kv_slot >= nkv)
            return failw(MESH_ATTN_ERR_INVALID, who, "block slot out of range");
        if (b.q_part < 0 || b.kv_part < 0)
            return failw(MESH_ATTN_ERR_INVALID, who, "negative partition id");
        if (b.kind < MESH_ATTN_FULL || b.kind > MESH_ATTN_SKIP)
            return failw(MESH_ATTN_ERR_INVALID, who, "block kind out of range");
        if (kind[b.q_slot][b.kv_slot] != -1)
            return failw(MESH_ATTN_ERR_INVALID, who, "duplicated (q_slot, kv_slot) block");
        if (q_part_of[b.q_slot] != -1 && q_part_of[b.q_slot] != b.q_part)
            return failw(MESH_ATTN_ERR_INVALID, who, "q_slot listed with two partitions");
        if (kv_part_of[b.kv_slot] != -1 && kv_part_of[b.kv_slot] != b.kv_part)
            return failw(MESH_ATTN_ERR_INVALID, who, "kv_slot listed with two partitions");
        if (b.kind == MESH_ATTN_DIAG && b.q_part != b.kv_part)
            return failw(MESH_ATTN_ERR_INVALID, who, "DIAG block with q_part != kv_part");
        kind[b.q_slot][b.kv_slot] = static_cast<int8_t>(b.kind);
        q_part_of[b.q_slot] = b.q_part;
        kv_part_of[b.kv_slot] = b.kv_part;
    }
    for (int a = 0; a < nq; ++a)
        for (int b = a + 1; b < nq; ++b)
            if (q_part_of[a] != -1 && q_part_of[a] == q_part_of[b])
                return failw(MESH_ATTN_ERR_INVALID, who, "two Q slots hold one partition");
    for (int a = 0; a < nkv; ++a)
        for (int b = a + 1; b < nkv; ++b)
            if (kv_part_of[a] != -1 && kv_part_of[a] == kv_part_of[b])
                return failw(MESH_ATTN_ERR_INVALID, who, "two KV slots hold one partition");

    // Pack non-SKIP entries per Q slot in KV-slot order; weigh each Q slot.
    int cost2[kMaxQSlots];  // 2 per FULL, 1 per DIAG
    int off = 0;
    for (int s = 0; s < nq; ++s) {
        qs.blk_off[s] = static_cast<uint16_t>(off);
        cost2[s] = 0;
        for (int j = 0; j < nkv; ++j) {
            const int kd = kind[s][j];
            if (kd == MESH_ATTN_FULL || kd == MESH_ATTN_DIAG) {
                qs.blk[off++] = static_cast<uint8_t>((j << 2) | kd);
                cost2[s] += kd == MESH_ATTN_FULL ? 2 : 1;
            }
        }
    }
    qs.blk_off[nq] = static_cast<uint16_t>(off);
    int order[kMaxQSlots];
    for (int s = 0; s < nq; ++s) order[s] = s;
    std::stable_sort(order, order + nq, [&](int a, int b) { return cost2[a] > cost2[b]; });
    for (int s = 0; s < nq; ++s) qs.q_order[s] = static_cast<uint8_t>(order[s]);

    if (ks != nullptr) {
        off = 0;
        for (int j = 0; j < nkv; ++j) {
            ks->blk_off[j] = static_cast<uint16_t>(off);
            for (int s = 0; s < nq; ++s) {
                const int kd = kind[s][j];
                if (kd == MESH_ATTN_FULL || kd == MESH_ATTN_DIAG)
                    ks->blk[off++] = static_cast<uint8_t>((s << 2) | kd);
            }
        }
        ks->blk_off[nkv] = static_cast<uint16_t>(off);
    }
    return MESH_ATTN_OK;
}

// Checks the shape fields of a tile description (not the block list).
static int check_tile_shape(const char* who, const mesh_attn_tile_desc& d) {
    if (d.dtype != MESH_ATTN_BF16 && d.dtype != MESH_ATTN_F32)
        return failw(MESH_ATTN_ERR_INVALID, who, "unknown dtype");
    if (d.part_len < 1) return failw(MESH_ATTN_ERR_INVALID, who, "part_len must be >= 1");
    if (d.n_q_slots < 1 || d.n_q_slots > MESH_ATTN_MAX_Q_SLOTS)
        return failw(MESH_ATTN_ERR_INVALID, who, "n_q_slots out of range");
    if (d.n_kv_slots < 1 || d.n_kv_slots > MESH_ATTN_MAX_KV_SLOTS)
        return failw(MESH_ATTN_ERR_INVALID, who, "n_kv_slots out of range");
    if (d.heads_q < 1 || d.heads_kv < 1 || d.heads_q % d.heads_kv != 0)
        return failw(MESH_ATTN_ERR_INVALID, who, "heads_q must be a positive multiple of heads_kv");
    if (d.heads_q > MESH_ATTN_MAX_HEADS)
        return failw(MESH_ATTN_ERR_INVALID, who, "heads_q above MESH_ATTN_MAX_HEADS");
    if (d.head_dim < 1) return failw(MESH_ATTN_ERR_INVALID, who, "head_dim must be >= 1");
    if (!(isfinite(d.softmax_scale) && d.softmax_scale > 0.0f))
        return failw(MESH_ATTN_ERR_INVALID, who, "softmax_scale must be finite and > 0");
    // Element counts must stay addressable with 64-bit offsets and the token
    // index with 32-bit integers.
    const int64_t q_tokens = static_cast<int64_t>(d.n_q_slots) * d.part_len;
    const int64_t kv_tokens = static_cast<int64_t>(d.n_kv_slots) * d.part_len;
    if (q_tokens > INT32_MAX || kv_tokens > INT32_MAX ||
        q_tokens * d.heads_q > INT32_MAX || kv_tokens * d.heads_kv > INT32_MAX)
        return failw(MESH_ATTN_ERR_INVALID, who, "tile too large");
    return MESH_ATTN_OK;
}

// The forward's work decomposition over (Q slot, token block, KV head,
// query-head group) for workgroups of `waves` waves of `wave_rows` rows.
template <typename Params>
static void set_row_decomposition(Params& p, const mesh_attn_tile_desc& d, int waves, int wave_rows) {
    p.part_len = d.part_len;
    p.heads_q = d.heads_q;
    p.heads_kv = d.heads_kv;
    p.group = d.heads_q / d.heads_kv;
    p.heads_per_wg = gcd(p.group, waves);
    p.tok_groups = waves / p.heads_per_wg;
    p.wave_rows = wave_rows;
    const int wg_rows = p.wave_rows * p.tok_groups;
    p.n_tok_blocks = (d.part_len + wg_rows - 1) / wg_rows;
    p.n_head_groups = p.group / p.heads_per_wg;
    p.n_q_slots = d.n_q_slots;
}

}  // namespace mesh_attn

using namespace mesh_attn;

namespace mesh_attn {

int plan_tile_fwd(const char* who, const mesh_attn_tile_desc& d, TileParams& p) {
    const int shape_st = check_tile_shape(who, d);
    if (shape_st != MESH_ATTN_OK) return shape_st;
    const bool supported = (d.dtype == MESH_ATTN_BF16 && d.head_dim == 128) ||
                           (d.dtype == MESH_ATTN_F32 && (d.head_dim == 64 || d.head_dim == 128));
    if (!supported)
        return failw(MESH_ATTN_ERR_UNSUPPORTED, who, "dtype/head_dim combination not built");

    memset(&p, 0, sizeof(p));
    const int st = build_schedule(who, d, p.sched, nullptr);
    if (st != MESH_ATTN_OK) return st;
    set_row_decomposition(p, d, d.dtype == MESH_ATTN_BF16 ? kTileWavesBf16 : kTileWavesF32,
                          d.dtype == MESH_ATTN_BF16 ? kWaveRowsBf16 : kWaveRowsF32);
    p.scale_log2e = d.softmax_scale * 1.4426950408889634f;
    if (tile_fwd_grid(p) > INT32_MAX) return failw(MESH_ATTN_ERR_INVALID, who, "grid too large");
    return MESH_ATTN_OK;
}

int plan_tile_bwd(const char* who, const mesh_attn_tile_desc& d, BwdDqParams& pq, BwdDkvParams& pk) {
    const int shape_st = check_tile_shape(who, d);
    if (shape_st != MESH_ATTN_OK) return shape_st;
    if (!(d.dtype == MESH_ATTN_BF16 && d.head_dim == 128))
        return failw(MESH_ATTN_ERR_UNSUPPORTED, who, "dtype/head_dim combination not built");

    memset(&pq, 0, sizeof(pq));
    memset(&pk, 0, sizeof(pk));
    const int st = build_schedule(who, d, pq.sched, &pk.sched);
    if (st != MESH_ATTN_OK) return st;

    set_row_decomposition(pq, d, kBwdDqWaves, kBwdRowsPerWave);
    pq.scale = d.softmax_scale;
    pq.scale_log2e = d.softmax_scale * 1.4426950408889634f;

    pk.part_len = d.part_len;
    pk.heads_q = d.heads_q;
    pk.heads_kv = d.heads_kv;
    pk.group = d.heads_q / d.heads_kv;
    pk.n_kv_slots = d.n_kv_slots;
    const int keys_per_wg = kBwdDkvWaves * kBwdRowsPerWave;
    pk.n_key_blocks = (d.part_len + keys_per_wg - 1) / keys_per_wg;
    pk.scale = pq.scale;
    pk.scale_log2e = pq.scale_log2e;
    if (tile_fwd_grid(pq) > INT32_MAX || tile_bwd_dkdv_grid(pk) > INT32_MAX)
        return failw(MESH_ATTN_ERR_INVALID, who, "grid too large");
    return MESH_ATTN_OK;
}

}  // namespace mesh_attn

extern "C" int mesh_attn_tile_fwd(const mesh_attn_tile_desc* desc, const void* q, const void* k,
                                  const void* v, void* o, float* lse, void* hip_stream) {
    const char* who = "tile_fwd";
    if (desc == nullptr) return failw(MESH_ATTN_ERR_INVALID, who, "desc is NULL");
    const mesh_attn_tile_desc& d = *desc;
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr)
        return failw(MESH_ATTN_ERR_INVALID, who, "NULL tensor pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return failw(MESH_ATTN_ERR_INVALID, who, "tensor pointer not 16-byte aligned");
    if (!aligned4(lse)) return failw(MESH_ATTN_ERR_INVALID, who, "lse pointer not 4-byte aligned");
    TileParams p;
    const int st = plan_tile_fwd(who, d, p);
    if (st != MESH_ATTN_OK) return st;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;

    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    const hipError_t e = d.dtype == MESH_ATTN_BF16 ? launch_tile_fwd_bf16(p, d.head_dim, stream)
                                                   : launch_tile_fwd_f32(p, d.head_dim, stream);
    return hip_status(e, "tile_fwd: kernel launch failed");
}

extern "C" int mesh_attn_lse_merge(int32_t n_parts, int64_t rows, int32_t head_dim, int32_t dtype,
                                   const void* o_parts, const float* lse_parts, void* o_out,
                                   float* lse_out, void* hip_stream) {
    const char* who = "lse_merge";
    if (n_parts < 1 || n_parts > 64)
        return failw(MESH_ATTN_ERR_INVALID, who, "n_parts must be in 1..64");
    if (rows < 0) return failw(MESH_ATTN_ERR_INVALID, who, "rows must be >= 0");
    if (dtype != MESH_ATTN_BF16 && dtype != MESH_ATTN_F32)
        return failw(MESH_ATTN_ERR_INVALID, who, "unknown dtype");
    const int vec = dtype == MESH_ATTN_BF16 ? 8 : 4;
    if (head_dim < 8 || head_dim > 512 || head_dim % vec != 0)
        return failw(MESH_ATTN_ERR_INVALID, who, "head_dim must be a multiple of 8 (bf16) "
                                           "or 4 (f32) in 8..512");
    if (o_parts == nullptr || lse_parts == nullptr || o_out == nullptr)
        return failw(MESH_ATTN_ERR_INVALID, who, "NULL tensor pointer");
    if (!aligned16(o_parts) || !aligned16(o_out) ||
        (reinterpret_cast<uintptr_t>(lse_parts) & 3u) != 0 ||
        (lse_out != nullptr && (reinterpret_cast<uintptr_t>(lse_out) & 3u) != 0))
        return failw(MESH_ATTN_ERR_INVALID, who, "misaligned pointer");
    if (rows > (INT64_MAX / 64) / head_dim)
        return failw(MESH_ATTN_ERR_INVALID, who, "rows too large");
    if (rows == 0) {
        clear_error();
        return MESH_ATTN_OK;
    }
    const hipError_t e = launch_lse_merge(n_parts, rows, head_dim, dtype, o_parts, lse_parts,
                                          o_out, lse_out, static_cast<hipStream_t>(hip_stream));
    return hip_status(e, "lse_merge: kernel launch failed");
}

extern "C" const char* mesh_attn_status_string(int status) {
    switch (status) {
        case MESH_ATTN_OK: return "ok";
        case MESH_ATTN_ERR_INVALID: return "invalid argument";
        case MESH_ATTN_ERR_CAPACITY: return "output capacity too small";
        case MESH_ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
        case MESH_ATTN_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

extern "C" const char* mesh_attn_last_error(void) { return g_last_error.c_str(); }

extern "C" int32_t mesh_attn_version(void) { return 100; }

extern "C" int mesh_attn_bwd_delta(int64_t rows, int32_t head_dim, int32_t dtype, const void* o,
                                   const void* dout, float* delta, void* hip_stream) {
    const char* who = "bwd_delta";
    if (rows < 0) return failw(MESH_ATTN_ERR_INVALID, who, "rows must be >= 0");
    if (dtype != MESH_ATTN_BF16 && dtype != MESH_ATTN_F32)
        return failw(MESH_ATTN_ERR_INVALID, who, "unknown dtype");
    const int vec = dtype == MESH_ATTN_BF16 ? 8 : 4;
    if (head_dim < 8 || head_dim > 512 || head_dim % vec != 0)
        return failw(MESH_ATTN_ERR_INVALID, who,
                     "head_dim must be a multiple of 8 (bf16) or 4 (f32) in 8..512");
    if (o == nullptr || dout == nullptr || delta == nullptr)
        return failw(MESH_ATTN_ERR_INVALID, who, "NULL tensor pointer");
    if (!aligned16(o) || !aligned16(dout) || (reinterpret_cast<uintptr_t>(delta) & 3u) != 0)
        return failw(MESH_ATTN_ERR_INVALID, who, "misaligned pointer");
    if (rows > (INT64_MAX / 64) / head_dim) return failw(MESH_ATTN_ERR_INVALID, who, "rows too large");
    if (rows == 0) {
        clear_error();
        return MESH_ATTN_OK;
    }
    const hipError_t e = launch_bwd_delta(rows, head_dim, dtype, o, dout, delta,
                                          static_cast<hipStream_t>(hip_stream));
    return hip_status(e, "bwd_delta: kernel launch failed");
}

extern "C" int mesh_attn_tile_bwd(const mesh_attn_tile_desc* desc, const void* q, const void* k,
                                  const void* v, const void* dout, const float* lse,
                                  const float* delta, float* dq, float* dk, float* dv,
                                  void* hip_stream) {
    const char* who = "tile_bwd";
    if (desc == nullptr) return failw(MESH_ATTN_ERR_INVALID, who, "desc is NULL");
    const mesh_attn_tile_desc& d = *desc;
    if (q == nullptr || k == nullptr || v == nullptr || dout == nullptr || lse == nullptr ||
        delta == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
        return failw(MESH_ATTN_ERR_INVALID, who, "NULL tensor pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv))
        return failw(MESH_ATTN_ERR_INVALID, who, "tensor pointer not 16-byte aligned");
    if (!aligned4(lse) || !aligned4(delta))
        return failw(MESH_ATTN_ERR_INVALID, who, "lse or delta pointer not 4-byte aligned");
    BwdDqParams pq;
    BwdDkvParams pk;
    const int st = plan_tile_bwd(who, d, pq, pk);
    if (st != MESH_ATTN_OK) return st;
    pq.q = q;
    pq.k = k;
    pq.v = v;
    pq.dout = dout;
    pq.lse = lse;
    pq.delta = delta;
    pq.dq = dq;
    pk.q = q;
    pk.k = k;
    pk.v = v;
    pk.dout = dout;
    pk.lse = lse;
    pk.delta = delta;
    pk.dk = dk;
    pk.dv = dv;

    const hipError_t e = launch_tile_bwd_bf16(pq, pk, d.head_dim, static_cast<hipStream_t>(hip_stream));
    return hip_status(e, "tile_bwd: kernel launch failed");
}
