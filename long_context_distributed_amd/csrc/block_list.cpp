// mesh_attn_block_list: the blocks of the Q-KV interaction matrix one mesh GPU
// owns.  Pure host code.
//
// Tutorial page on Mesh-Attention, section "From 1-D ring to 2-D mesh": rows of
// the matrix are Q partitions, columns are KV partitions; each GPU gets a 2-D
// tile and only talks to its mesh row (for Q) and mesh column (for KV); the
// figure's panel (c) rotates the KV block indices so that each GPU works on
// its own data.  The arXiv abstract (mlsanity page) names this KV Partition
// Rotation.  The exact rotation is not printed; the reading used here is that
// GPU (r, c) visits its column starting with its own partition and stepping
// down cyclically, which keeps every property the pages state (own block in
// the tile, column-only KV peers, each rotation step a permutation of
// senders).
#include "mesh_attn.h"

#include "status.h"

extern "C" int mesh_attn_block_list(int32_t mesh_rows, int32_t mesh_cols, int32_t row,
                                    int32_t col, int32_t causal, int32_t kv_rotate,
                                    mesh_attn_block* out, int32_t capacity, int32_t* n_out) {
    using mesh_attn::fail;
    if (n_out == nullptr) return fail(MESH_ATTN_ERR_INVALID, "block_list: n_out is NULL");
    if (mesh_rows < 1 || mesh_cols < 1)
        return fail(MESH_ATTN_ERR_INVALID, "block_list: mesh dimensions must be >= 1");
    if (static_cast<int64_t>(mesh_rows) * mesh_cols > 65536)
        return fail(MESH_ATTN_ERR_INVALID, "block_list: mesh larger than 65536 GPUs");
    if (row < 0 || row >= mesh_rows || col < 0 || col >= mesh_cols)
        return fail(MESH_ATTN_ERR_INVALID, "block_list: tile position outside the mesh");

    const int64_t count = static_cast<int64_t>(mesh_rows) * mesh_cols;
    *n_out = static_cast<int32_t>(count);
    if (out == nullptr || capacity < count)
        return fail(MESH_ATTN_ERR_CAPACITY, "block_list: output capacity too small");

    int32_t i = 0;
    for (int32_t kv_slot = 0; kv_slot < mesh_rows; ++kv_slot) {
        const int32_t kv_part = kv_rotate ? ((row + kv_slot) % mesh_rows) * mesh_cols + col
                                          : col * mesh_rows + kv_slot;
        for (int32_t q_slot = 0; q_slot < mesh_cols; ++q_slot) {
            const int32_t q_part = row * mesh_cols + q_slot;
            int32_t kind = MESH_ATTN_FULL;
            if (causal) {
                kind = kv_part < q_part ? MESH_ATTN_FULL
                                        : (kv_part == q_part ? MESH_ATTN_DIAG : MESH_ATTN_SKIP);
            }
            out[i++] = mesh_attn_block{q_slot, kv_slot, q_part, kv_part, kind};
        }
    }
    mesh_attn::clear_error();
    return MESH_ATTN_OK;
}
