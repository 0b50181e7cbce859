// Greedy communication/computation plan of one mesh GPU (host code).
//
// Mesh-Attention tutorial page, section "Greedy algorithm": the next
// communication is the one that unlocks the most compute blocks, and ready
// compute is held back to fill later waits on communication rather than run
// as soon as its data arrives.  The step model is the ring's "compute one
// step, transfer one step" generalised to the tile: each step runs at most
// one transfer beside a set of ready blocks and lasts as long as the longer
// of the two.
//
// Transfers of GPU (r, c): the Q partition of each Q slot it does not hold,
// the KV partition of each KV slot it does not hold (only slots some non-SKIP
// block needs), and, once a row's non-SKIP blocks are computed, the partial
// output of every Q slot whose partition belongs to another GPU.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "mesh_attn.h"
#include "status.h"

namespace {

struct Op {
    int kind;  // MESH_ATTN_COMM_*
    int slot;
};

struct PlanState {
    int R, C, g;
    std::vector<mesh_attn_block> need;  // non-SKIP blocks, block-list order
    std::vector<int> q_part, kv_part;    // by slot
    std::vector<char> q_have, kv_have;   // data present
    std::vector<char> computed;          // by index into need
};

int row_left(const PlanState& st, int s) {
    int n = 0;
    for (size_t i = 0; i < st.need.size(); ++i)
        if (st.need[i].q_slot == s && !st.computed[i]) ++n;
    return n;
}

// Blocks a receive makes computable, given what is present now.
int unlocked_by(const PlanState& st, const Op& op) {
    int n = 0;
    for (const mesh_attn_block& b : st.need) {
        if (op.kind == MESH_ATTN_COMM_RECV_KV && b.kv_slot == op.slot && st.q_have[b.q_slot]) ++n;
        if (op.kind == MESH_ATTN_COMM_RECV_Q && b.q_slot == op.slot && st.kv_have[b.kv_slot]) ++n;
    }
    return n;
}

// Non-SKIP blocks on the receive's row or column.
int blocks_on(const PlanState& st, const Op& op) {
    int n = 0;
    for (const mesh_attn_block& b : st.need)
        if ((op.kind == MESH_ATTN_COMM_RECV_KV ? b.kv_slot : b.q_slot) == op.slot) ++n;
    return n;
}

double block_seconds(const mesh_attn_block& b, const mesh_attn_plan_costs& c) {
    return b.kind == MESH_ATTN_FULL ? c.full_block_s : c.diag_block_s;
}

double comm_seconds(int kind, const mesh_attn_plan_costs& c) {
    switch (kind) {
        case MESH_ATTN_COMM_RECV_Q: return c.recv_q_s;
        case MESH_ATTN_COMM_RECV_KV: return c.recv_kv_s;
        case MESH_ATTN_COMM_SEND_O: return c.send_o_s;
        default: return 0.0;
    }
}

bool valid_cost(double x) { return isfinite(x) && x >= 0.0; }

}  // namespace

static int plan_impl(int32_t mesh_rows, int32_t mesh_cols, int32_t row, int32_t col, int32_t causal,
                     int32_t kv_rotate, const mesh_attn_plan_costs* costs, mesh_attn_plan_step* steps,
                     int32_t step_capacity, int32_t* n_steps, mesh_attn_block* order, int32_t order_capacity,
                     int32_t* n_order) {
    using mesh_attn::fail;
    if (costs == nullptr) return fail(MESH_ATTN_ERR_INVALID, "plan: costs is NULL");
    if (n_steps == nullptr || n_order == nullptr)
        return fail(MESH_ATTN_ERR_INVALID, "plan: n_steps and n_order must not be NULL");
    if (mesh_rows > MESH_ATTN_MAX_KV_SLOTS || mesh_cols > MESH_ATTN_MAX_Q_SLOTS)
        return fail(MESH_ATTN_ERR_INVALID, "plan: a tile of this mesh exceeds the slot limits");
    const mesh_attn_plan_costs& cs = *costs;
    if (!valid_cost(cs.recv_q_s) || !valid_cost(cs.recv_kv_s) || !valid_cost(cs.send_o_s) ||
        !valid_cost(cs.full_block_s) || !valid_cost(cs.diag_block_s))
        return fail(MESH_ATTN_ERR_INVALID, "plan: costs must be finite and >= 0");
    if (cs.delay != 0 && cs.delay != 1) return fail(MESH_ATTN_ERR_INVALID, "plan: delay must be 0 or 1");

    int32_t nb = 0;
    {
        const int st = mesh_attn_block_list(mesh_rows, mesh_cols, row, col, causal, kv_rotate, nullptr, 0, &nb);
        if (st != MESH_ATTN_ERR_CAPACITY) return st;  // invalid geometry (message already set)
    }
    std::vector<mesh_attn_block> blocks(nb);
    {
        int32_t n2 = 0;
        const int st = mesh_attn_block_list(mesh_rows, mesh_cols, row, col, causal, kv_rotate, blocks.data(),
                                            nb, &n2);
        if (st != MESH_ATTN_OK) return st;
    }

    PlanState st;
    st.R = mesh_rows;
    st.C = mesh_cols;
    st.g = row * mesh_cols + col;
    st.q_part.assign(mesh_cols, -1);
    st.kv_part.assign(mesh_rows, -1);
    for (const mesh_attn_block& b : blocks) {
        st.q_part[b.q_slot] = b.q_part;
        st.kv_part[b.kv_slot] = b.kv_part;
        if (b.kind != MESH_ATTN_SKIP) st.need.push_back(b);
    }
    st.q_have.assign(mesh_cols, 0);
    st.kv_have.assign(mesh_rows, 0);
    for (int s = 0; s < mesh_cols; ++s) st.q_have[s] = st.q_part[s] == st.g;
    for (int j = 0; j < mesh_rows; ++j) st.kv_have[j] = st.kv_part[j] == st.g;
    st.computed.assign(st.need.size(), 0);

    std::vector<char> row_used(mesh_cols, 0), col_used(mesh_rows, 0);
    for (const mesh_attn_block& b : st.need) {
        row_used[b.q_slot] = 1;
        col_used[b.kv_slot] = 1;
    }
    std::vector<Op> pending;
    for (int j = 0; j < mesh_rows; ++j)
        if (col_used[j] && !st.kv_have[j]) pending.push_back({MESH_ATTN_COMM_RECV_KV, j});
    for (int s = 0; s < mesh_cols; ++s)
        if (row_used[s] && !st.q_have[s]) pending.push_back({MESH_ATTN_COMM_RECV_Q, s});
    std::vector<int> sends;  // Q slots whose partial goes back to their owner, in slot order
    for (int s = 0; s < mesh_cols; ++s)
        if (row_used[s] && st.q_part[s] != st.g) sends.push_back(s);

    std::vector<mesh_attn_plan_step> out_steps;
    std::vector<mesh_attn_block> out_order;
    size_t n_done = 0;
    double t = 0.0;
    while (!pending.empty() || !sends.empty() || n_done < st.need.size()) {
        // Rule 1: the transfer of this step.
        int first_ready_send = -1;
        for (int s : sends)
            if (row_left(st, s) == 0) {
                first_ready_send = s;
                break;
            }
        Op op{MESH_ATTN_COMM_NONE, -1};
        if (!pending.empty()) {
            size_t bi = 0;
            int bu = -1, bp = -1;
            for (size_t i = 0; i < pending.size(); ++i) {
                const int u = unlocked_by(st, pending[i]);
                const int pot = blocks_on(st, pending[i]);
                const Op& a = pending[i];
                const Op& b = pending[bi];
                bool better;
                if (bu < 0) better = true;
                else if (u != bu) better = u > bu;
                else if (pot != bp) better = pot > bp;
                else if (a.kind != b.kind) better = a.kind == MESH_ATTN_COMM_RECV_Q;
                else better = a.slot < b.slot;
                if (better) {
                    bi = i;
                    bu = u;
                    bp = pot;
                }
            }
            if (bu == 0 && first_ready_send >= 0) op = {MESH_ATTN_COMM_SEND_O, first_ready_send};
            else op = pending[bi];
        } else if (first_ready_send >= 0) {
            op = {MESH_ATTN_COMM_SEND_O, first_ready_send};
        }
        const double comm_s = comm_seconds(op.kind, cs);

        // Rule 2: the blocks computed beside it.
        std::vector<int> ready;
        std::vector<int> left_at(mesh_cols, 0);
        for (int s = 0; s < mesh_cols; ++s) left_at[s] = row_left(st, s);
        for (size_t i = 0; i < st.need.size(); ++i) {
            const mesh_attn_block& b = st.need[i];
            if (!st.computed[i] && st.q_have[b.q_slot] && st.kv_have[b.kv_slot]) ready.push_back((int)i);
        }
        std::sort(ready.begin(), ready.end(), [&](int x, int y) {
            const mesh_attn_block& a = st.need[x];
            const mesh_attn_block& b = st.need[y];
            const int la = st.q_part[a.q_slot] == st.g, lb = st.q_part[b.q_slot] == st.g;
            if (la != lb) return la < lb;  // rows to be sent first
            if (left_at[a.q_slot] != left_at[b.q_slot]) return left_at[a.q_slot] < left_at[b.q_slot];
            if (a.q_slot != b.q_slot) return a.q_slot < b.q_slot;
            return a.kv_slot < b.kv_slot;
        });
        size_t take = 0;
        if (cs.delay == 0) {
            take = ready.size();
        } else if (op.kind != MESH_ATTN_COMM_NONE) {
            double acc = 0.0;
            while (take < ready.size() && acc < comm_s) acc += block_seconds(st.need[ready[take++]], cs);
        } else if (!sends.empty()) {
            // No transfer possible: finish the next row whose partial is to be sent.
            if (!ready.empty()) {
                const int target = st.need[ready[0]].q_slot;
                int remaining = left_at[target];
                while (take < ready.size() && remaining > 0) {
                    if (st.need[ready[take]].q_slot == target) --remaining;
                    ++take;
                }
            }
        } else {
            take = ready.size();
        }
        mesh_attn_plan_step step;
        memset(&step, 0, sizeof(step));
        step.comm = op.kind;
        step.slot = op.slot;
        step.block_begin = static_cast<int32_t>(out_order.size());
        step.block_count = static_cast<int32_t>(take);
        double compute_s = 0.0;
        for (size_t k = 0; k < take; ++k) {
            const int i = ready[k];
            compute_s += block_seconds(st.need[i], cs);
            st.computed[i] = 1;
            out_order.push_back(st.need[i]);
        }
        n_done += take;
        step.comm_s = comm_s;
        step.compute_s = compute_s;
        step.start_s = t;
        t += std::max(comm_s, compute_s);
        step.end_s = t;
        out_steps.push_back(step);

        if (op.kind == MESH_ATTN_COMM_RECV_KV || op.kind == MESH_ATTN_COMM_RECV_Q) {
            if (op.kind == MESH_ATTN_COMM_RECV_KV) st.kv_have[op.slot] = 1;
            else st.q_have[op.slot] = 1;
            for (size_t i = 0; i < pending.size(); ++i)
                if (pending[i].kind == op.kind && pending[i].slot == op.slot) {
                    pending.erase(pending.begin() + i);
                    break;
                }
        } else if (op.kind == MESH_ATTN_COMM_SEND_O) {
            sends.erase(std::find(sends.begin(), sends.end(), op.slot));
        } else if (take == 0) {
            return fail(MESH_ATTN_ERR_INVALID, "plan: internal error, no progress");
        }
    }

    *n_steps = static_cast<int32_t>(out_steps.size());
    *n_order = static_cast<int32_t>(out_order.size());
    if (steps == nullptr || order == nullptr || step_capacity < *n_steps || order_capacity < *n_order)
        return fail(MESH_ATTN_ERR_CAPACITY, "plan: output arrays too small (counts written)");
    std::copy(out_steps.begin(), out_steps.end(), steps);
    std::copy(out_order.begin(), out_order.end(), order);
    mesh_attn::clear_error();
    return MESH_ATTN_OK;
}

extern "C" int mesh_attn_plan(int32_t mesh_rows, int32_t mesh_cols, int32_t row, int32_t col,
                              int32_t causal, int32_t kv_rotate, const mesh_attn_plan_costs* costs,
                              mesh_attn_plan_step* steps, int32_t step_capacity, int32_t* n_steps,
                              mesh_attn_block* order, int32_t order_capacity, int32_t* n_order) {
    // No exception crosses the C ABI (the only source is host memory exhaustion).
    try {
        return plan_impl(mesh_rows, mesh_cols, row, col, causal, kv_rotate, costs, steps, step_capacity,
                         n_steps, order, order_capacity, n_order);
    } catch (...) {
        return mesh_attn::fail(MESH_ATTN_ERR_INVALID, "plan: out of host memory");
    }
}
