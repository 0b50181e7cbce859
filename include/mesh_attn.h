/*
 * mesh_attn.h - C ABI of the Mesh-Attention tile library for AMD MI355X (gfx950).
 *
 * One GPU of Mesh-Attention owns a 2-D tile of the Q-KV interaction matrix:
 * a set of Q sequence partitions (its mesh row's) against a set of KV
 * partitions (its mesh column's, in KV-Partition-Rotation order).  It computes
 * blockwise softmax attention over the tile, producing a partial output and a
 * log-sum-exp per query row, and the owner of a Q partition combines the
 * partial results returned by its mesh-row peers with a log-sum-exp merge.
 *
 * Sources (pages on Mesh-Attention and on ring attention):
 *   - Mesh-Attention tutorial page ("Mesh-Attention: A New Communication-
 *     Efficient Distributed Attention with Improved Data Locality"), section
 *     "From 1-D ring to 2-D mesh" with figure panels (b) and (c): the Q-KV
 *     matrix, 2-D tiles, row/column peers, index rotation of KV blocks;
 *     section on the greedy algorithm: partial outputs travel back to the
 *     Q owner.
 *   - mlsanity page for arXiv 2512.20968, section "Abstract (arXiv)": each GPU
 *     collects only subsets of the Q and KV partitions; KV Partition Rotation.
 *   - Ring-attention page ("环形注意力：突破长序列处理瓶颈的分布式计算范式"),
 *     sections on log-sum-exp numerical stability (running max m and exponent
 *     sum l) and on the decomposition of attention over KV blocks (printed
 *     without the log-sum-exp weights; the merge below uses the weighted form).
 *
 * Conventions
 *   - All integers are int32_t unless stated.  Tensors are dense, row-major,
 *     token-major.  Device pointers to bf16/f32 row data (q, k, v, o, dout,
 *     partial and merged outputs, gradients) must be 16-byte aligned; the
 *     per-row float32 arrays (lse, lse_parts, lse_out, delta) 4-byte aligned,
 *     so that a tile's lse may be written straight into one slot of a
 *     merge's [n, rows] lse array whatever rows is.
 *   - Device buffers and the stream belong to the caller.  The library
 *     allocates no device memory and keeps no state between calls except a
 *     thread-local text of the last error (mesh_attn_last_error).
 *   - Every call validates its arguments on the host before any HIP call and
 *     returns a status code; invalid arguments launch nothing.  Kernels run
 *     asynchronously on the given stream (NULL = the default stream); a fault
 *     inside a kernel surfaces at the caller's next synchronisation.
 *   - Outputs must not alias inputs.  Calls are thread-safe.
 */
#ifndef MESH_ATTN_H
#define MESH_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef MESH_ATTN_API
#define MESH_ATTN_API __attribute__((visibility("default")))
#endif

/* Status codes. */
enum {
    MESH_ATTN_OK = 0,
    MESH_ATTN_ERR_INVALID = -1,     /* an argument is out of range or inconsistent */
    MESH_ATTN_ERR_CAPACITY = -2,    /* output array too small; the needed count is reported */
    MESH_ATTN_ERR_UNSUPPORTED = -3, /* valid in principle but not built (dtype, head_dim) */
    MESH_ATTN_ERR_HIP = -4          /* the HIP runtime refused a launch */
};

/* Element types of Q, K, V and of the partial outputs. */
enum { MESH_ATTN_BF16 = 0, MESH_ATTN_F32 = 1 };

/* Causal class of one (Q partition, KV partition) block.  With the rule
 * "a key is visible to a query when its position is not after the query's"
 * and equal-length contiguous partitions: FULL when kv_part < q_part (or for
 * any block of a non-causal tile), DIAG when kv_part == q_part (a key at
 * partition offset w is visible to the query at offset u iff w <= u), SKIP
 * when kv_part > q_part (no work, no memory traffic). */
enum { MESH_ATTN_FULL = 0, MESH_ATTN_DIAG = 1, MESH_ATTN_SKIP = 2 };

/* One block of a tile: Q slot q_slot (holding sequence partition q_part)
 * against KV slot kv_slot (holding partition kv_part). */
typedef struct {
    int32_t q_slot, kv_slot, q_part, kv_part, kind;
} mesh_attn_block;

/* Largest tile the library accepts. */
#define MESH_ATTN_MAX_Q_SLOTS 64
#define MESH_ATTN_MAX_KV_SLOTS 64
#define MESH_ATTN_MAX_BLOCKS 1024
/* Most query heads per tile (keeps a token row of every tensor under 2 MiB). */
#define MESH_ATTN_MAX_HEADS 4096

/*
 * mesh_attn_block_list - the blocks GPU (row, col) of a mesh_rows x mesh_cols
 * mesh owns (tutorial page, "From 1-D ring to 2-D mesh"; abstract on the
 * mlsanity page).
 *
 * GPU (r, c) has id g = r*mesh_cols + c and holds sequence partition g.
 *   Q slots:  partition r*mesh_cols + t for t = 0 .. mesh_cols-1 (its mesh row).
 *   KV slots: kv_rotate != 0: partition ((r + k) mod mesh_rows)*mesh_cols + c
 *             for k = 0 .. mesh_rows-1 - its mesh column, starting with its own
 *             partition and stepping down the column cyclically (the reading
 *             of KV Partition Rotation used here);
 *             kv_rotate == 0: partition c*mesh_rows + k (contiguous block tiling).
 *   kind:     as in the enum above when causal != 0; FULL otherwise.
 * Entries are written KV-slot major, then Q slot: mesh_cols*mesh_rows entries.
 *
 * out may be NULL to query the count.  If out is NULL or capacity is smaller
 * than the count, *n_out receives the count and MESH_ATTN_ERR_CAPACITY is
 * returned (nothing is written to out).  mesh_rows, mesh_cols >= 1,
 * mesh_rows*mesh_cols <= 65536, 0 <= row < mesh_rows, 0 <= col < mesh_cols,
 * else MESH_ATTN_ERR_INVALID.  Pure host code: needs no GPU.
 */
MESH_ATTN_API int mesh_attn_block_list(int32_t mesh_rows, int32_t mesh_cols, int32_t row, int32_t col,
                         int32_t causal, int32_t kv_rotate,
                         mesh_attn_block *out, int32_t capacity, int32_t *n_out);

/* Shape of one tile-forward call. */
typedef struct {
    int32_t dtype;          /* MESH_ATTN_BF16 or MESH_ATTN_F32 */
    int32_t part_len;       /* L: tokens per partition, >= 1 */
    int32_t n_q_slots;      /* Q partitions in the tile, 1 .. MESH_ATTN_MAX_Q_SLOTS */
    int32_t n_kv_slots;     /* KV partitions in the tile, 1 .. MESH_ATTN_MAX_KV_SLOTS */
    int32_t heads_q;        /* H_q, 1 .. MESH_ATTN_MAX_HEADS */
    int32_t heads_kv;       /* H_kv >= 1, divides H_q; query head h reads KV head h / (H_q/H_kv) */
    int32_t head_dim;       /* d: 128 for bf16; 64 or 128 for f32 */
    float softmax_scale;    /* finite and > 0; usually 1/sqrt(d) */
    const mesh_attn_block *blocks; /* host array, read during the call only */
    int32_t n_blocks;       /* 0 .. MESH_ATTN_MAX_BLOCKS */
} mesh_attn_tile_desc;

/*
 * mesh_attn_tile_fwd - blockwise softmax attention of one tile (tutorial page,
 * "From 1-D ring to 2-D mesh"; the per-row running maximum and exponent sum of
 * the ring-attention page's log-sum-exp section).
 *
 *   q   [n_q_slots*L, H_q, d]   Q slot s holds tokens s*L .. s*L+L-1
 *   k,v [n_kv_slots*L, H_kv, d] KV slot j holds tokens j*L .. j*L+L-1
 *   o   [n_q_slots*L, H_q, d]   output, same dtype as q
 *   lse [n_q_slots*L, H_q]      float32
 *
 * For query row (token i of Q slot s, head h) the visible keys are the union,
 * over the listed blocks (s, j) whose kind is not SKIP, of the keys of KV slot
 * j - all of them for FULL, offsets w <= u for DIAG (u = i's offset in its
 * partition).  With scores x = softmax_scale * q.k over the visible keys:
 *   o = sum softmax(x) v,  lse = ln(sum exp(x))   (natural log, scaled scores)
 * A row with no visible key gets o = 0 and lse = -inf.  Pairs (s, j) that
 * are not listed are treated as SKIP, so a subset of a tile's blocks can be
 * computed from the same buffers.
 *
 * Validation (MESH_ATTN_ERR_INVALID): NULL desc, pointers or blocks with
 * n_blocks > 0; misaligned pointers; sizes out of range; H_q % H_kv != 0;
 * softmax_scale not finite or <= 0; a block with a slot out of range, a kind
 * out of range, a duplicated (q_slot, kv_slot), a slot listed with two
 * different partitions, two slots holding the same partition, or a DIAG
 * block whose q_part != kv_part.  Unsupported dtype/head_dim pairs return
 * MESH_ATTN_ERR_UNSUPPORTED.  hip_stream is a hipStream_t.
 */
MESH_ATTN_API int mesh_attn_tile_fwd(const mesh_attn_tile_desc *desc, const void *q, const void *k,
                       const void *v, void *o, float *lse, void *hip_stream);

/*
 * mesh_attn_lse_merge - combine n_parts partial results of the same query
 * rows (tutorial page, greedy-algorithm section: partial outputs return to
 * the Q owner; ring-attention page, log-sum-exp section).  Per row:
 *   M = max_i lse_i; if M = -inf: o = 0, lse = -inf;
 *   else w_i = exp(lse_i - M), o = sum_i w_i o_i / sum_i w_i,
 *        lse = M + ln(sum_i w_i).
 * A partial with lse_i = -inf contributes nothing and its output row is not
 * read.  Accumulation is in float32; o is written in dtype.
 *
 *   o_parts   [n_parts, rows, head_dim] (dtype)    lse_parts [n_parts, rows] float32
 *   o_out     [rows, head_dim] (dtype)             lse_out   [rows] float32, may be NULL
 *
 * rows is usually tokens*H_q.  n_parts 1..64, rows >= 0 (0 launches
 * nothing), head_dim a multiple of 8 (bf16) or 4 (f32) between 8 and 512.
 */
MESH_ATTN_API int mesh_attn_lse_merge(int32_t n_parts, int64_t rows, int32_t head_dim, int32_t dtype,
                        const void *o_parts, const float *lse_parts, void *o_out,
                        float *lse_out, void *hip_stream);

/*
 * mesh_attn_bwd_delta - per-row D = sum_d dout * o, the term the attention
 * backward subtracts in dS = P (dP - D).  The pages aim the method at
 * long-context training (tutorial page, the greedy-scheduling section and
 * the closing summary) but give no backward formula; this library takes the
 * plain derivative of softmax attention.
 *
 *   o, dout [rows, head_dim] (dtype)      delta [rows] float32
 *
 * o is the rows' final (merged) output.  rows >= 0 (0 launches nothing);
 * head_dim a multiple of 8 (bf16) or 4 (f32) between 8 and 512.  The dot
 * product is accumulated in float32.
 */
MESH_ATTN_API int mesh_attn_bwd_delta(int64_t rows, int32_t head_dim, int32_t dtype, const void *o,
                        const void *dout, float *delta, void *hip_stream);

/*
 * mesh_attn_tile_bwd - one tile's share of the attention gradients (same
 * tile description and visibility rules as mesh_attn_tile_fwd).  For every
 * visible pair of query row i (token, head h) and key j (KV head h / G) with
 * s_ij = softmax_scale * q_i.k_j:
 *   P_ij = exp(s_ij - lse_i)           lse_i: the row's final lse, natural log
 *   dv_j += P_ij dout_i
 *   dS_ij = P_ij (dout_i.v_j - delta_i)
 *   dq_i += softmax_scale dS_ij k_j,   dk_j += softmax_scale dS_ij q_i
 * Summed over all tiles of the mesh these are the gradients of full
 * attention; a Q (KV) owner adds the dq (dk, dv) shares its peers return.
 * A row with lse = -inf contributes nothing.
 *
 *   q, dout [n_q_slots*L, H_q, d] (dtype)   lse, delta [n_q_slots*L, H_q] float32
 *   k, v    [n_kv_slots*L, H_kv, d] (dtype)
 *   dq      [n_q_slots*L, H_q, d] float32   (written, not accumulated)
 *   dk, dv  [n_kv_slots*L, H_kv, d] float32 (written, not accumulated)
 * Rows of dq, dk and dv that no visible pair reaches are written as 0.
 * Validation as for mesh_attn_tile_fwd (messages say "tile_bwd"); built for
 * bf16 with d = 128, anything else returns MESH_ATTN_ERR_UNSUPPORTED.
 */
MESH_ATTN_API int mesh_attn_tile_bwd(const mesh_attn_tile_desc *desc, const void *q, const void *k,
                       const void *v, const void *dout, const float *lse, const float *delta,
                       float *dq, float *dk, float *dv, void *hip_stream);

/* Transfers of a plan step (mesh_attn_plan). */
enum {
    MESH_ATTN_COMM_NONE = 0,    /* no transfer in this step */
    MESH_ATTN_COMM_RECV_Q = 1,  /* receive the Q partition of Q slot `slot` */
    MESH_ATTN_COMM_RECV_KV = 2, /* receive the K and V partition of KV slot `slot` */
    MESH_ATTN_COMM_SEND_O = 3   /* send the partial output (O, lse) of Q slot `slot` to its owner */
};

/* Costs of the plan's step model, in seconds (finite, >= 0).  A caller
 * derives them from its shapes: a Q partition is L*H_q*d*s bytes, a KV
 * partition 2*L*H_kv*d*s, a partial output L*H_q*(d*s + 4) (s = bytes per
 * element), each over the link's bandwidth; a FULL block is 4*L*L*d*H_q
 * flops and a DIAG block 4*L*(L+1)/2*d*H_q, each over the tile kernel's
 * measured rate. */
typedef struct {
    double recv_q_s;      /* receive one Q partition */
    double recv_kv_s;     /* receive one KV partition (K and V) */
    double send_o_s;      /* send one partial output */
    double full_block_s;  /* compute one FULL block */
    double diag_block_s;  /* compute one DIAG block */
    int32_t delay;        /* 1: hold ready blocks back to fill later transfers (the
                           * greedy rule); 0: compute every ready block at once */
} mesh_attn_plan_costs;

/* One step of a plan: a transfer beside a run of blocks of `order`. */
typedef struct {
    int32_t comm;         /* MESH_ATTN_COMM_* */
    int32_t slot;         /* Q slot (RECV_Q, SEND_O) or KV slot (RECV_KV); -1 for NONE */
    int32_t block_begin;  /* the step computes order[block_begin .. block_begin+block_count) */
    int32_t block_count;
    double comm_s;        /* the transfer's time */
    double compute_s;     /* the blocks' time */
    double start_s;       /* simulated start: the previous step's end (0 for the first) */
    double end_s;         /* start_s + max(comm_s, compute_s) */
} mesh_attn_plan_step;

/*
 * mesh_attn_plan - the greedy communication/computation schedule of GPU
 * (row, col) of a mesh_rows x mesh_cols mesh (tutorial page, section
 * "Greedy algorithm"; greedy scheduling in the abstract on the mlsanity
 * page).  Pure host code: needs no GPU.
 *
 * The tile is mesh_attn_block_list(mesh_rows, mesh_cols, row, col, causal,
 * kv_rotate).  The GPU holds partition row*mesh_cols + col from the start;
 * a non-SKIP block can be computed once its Q slot's and KV slot's
 * partitions are present.  Transfers: receive each Q or KV partition some
 * non-SKIP block needs and the GPU does not hold, and send back the partial
 * output of each Q slot that belongs to another GPU once that row's
 * non-SKIP blocks are computed.  Steps run in lock-step: each runs at most
 * one transfer beside a set of ready blocks and lasts max(transfer,
 * compute); data received in a step is usable from the next step.
 *   Transfer choice: the pending receive that makes the most blocks
 *     computable; ties to the one whose slot has more non-SKIP blocks, then
 *     Q before KV, then the lower slot.  Sends follow the receives (one goes
 *     earlier only if no pending receive unlocks anything), ready sends in
 *     slot order.
 *   Compute choice (delay = 1): ready blocks in priority order until their
 *     time covers the step's transfer; the rest wait.  Priority: rows whose
 *     partial is sent first, rows with fewer blocks left first, then Q slot,
 *     then KV slot.  A step with no transfer possible finishes the next row
 *     to be sent (or, with no send left, computes everything that remains).
 *     delay = 0 computes every ready block at once.
 *
 * Outputs: steps[0 .. *n_steps) and order[0 .. *n_order), the non-SKIP
 * blocks in compute order (block-list tuples).  The makespan is
 * steps[*n_steps - 1].end_s (0 steps for a tile with no work and no
 * transfer).  If steps or order is NULL or a capacity is too small, the two
 * counts are written and MESH_ATTN_ERR_CAPACITY is returned (nothing else is
 * written): a size query.  MESH_ATTN_ERR_INVALID: NULL costs, n_steps or
 * n_order; a cost not finite or negative; delay not 0 or 1; mesh_rows > 64
 * or mesh_cols > 64 (the tile limits); anything mesh_attn_block_list
 * rejects; host memory exhausted while planning (the last-error text says
 * so).  No C++ exception leaves the call.
 */
MESH_ATTN_API int mesh_attn_plan(int32_t mesh_rows, int32_t mesh_cols, int32_t row, int32_t col,
                   int32_t causal, int32_t kv_rotate, const mesh_attn_plan_costs *costs,
                   mesh_attn_plan_step *steps, int32_t step_capacity, int32_t *n_steps,
                   mesh_attn_block *order, int32_t order_capacity, int32_t *n_order);

/* Text of a status code (static storage). */
MESH_ATTN_API const char *mesh_attn_status_string(int status);

/* Text describing the last failed call on this thread ("" if none). */
MESH_ATTN_API const char *mesh_attn_last_error(void);

/* Library version, e.g. 100 for 0.1.0. */
MESH_ATTN_API int32_t mesh_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MESH_ATTN_H */
