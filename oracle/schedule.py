"""Oracle: the greedy communication/computation schedule of one mesh GPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources:

* Mesh-Attention tutorial page, section "Greedy algorithm" (贪心算法): a GPU
  of the mesh receives Q partitions, KV partitions and partial outputs, and
  the space of schedules explodes; the pages' greedy algorithm (1) picks as
  the next communication the one that unlocks the most compute blocks, and
  (2) does not compute every block as soon as its data is there, but keeps
  some ready work in hand to fill later waits on communication.  The same
  section contrasts Ring-Attention's schedule: compute one step, transfer
  one step.
* mlsanity page for arXiv 2512.20968, "Abstract (arXiv)": greedy scheduling
  is what overlaps communication with computation.

Model (the pages give only the two rules; this is the plainest reading that
they and the Ring-Attention contrast support):

* One GPU (r, c) of an R x C mesh, its tile from ``block_list_ref``.  The
  GPU holds sequence partition g = r*C + c from the start.  A non-SKIP block
  (Q slot s, KV slot j) can be computed once Q slot s and KV slot j are both
  present (held from the start, or received).
* Transfers: receive the Q partition of a Q slot, receive the KV partition
  of a KV slot (only slots that some non-SKIP block needs), and send the
  partial output of a Q slot whose partition is not the GPU's own back to
  its owner, once every non-SKIP block of that slot's row is computed.
* Lock-step steps, as in the ring's "compute one step, transfer one step":
  each step runs at most one transfer beside a set of ready blocks, and
  lasts max(transfer time, sum of the blocks' times).  Data received in a
  step can be used from the next step on.  The makespan is the sum.
* Rule 1, choosing the transfer: among the pending receives, the one that
  unlocks the most blocks (blocks whose other side is already present);
  ties go to the one whose slot has more non-SKIP blocks in all, then to Q
  before KV (a Q partition opens a row whose partial must travel back, so
  its send can overlap later compute), then to the lower slot (for KV, the
  rotation order).  Partial-output sends unlock nothing, so they follow the
  receives; one is taken earlier only when no pending receive unlocks
  anything.  Ready sends go in slot order.
* Rule 2, delaying compute: a step with a transfer computes ready blocks,
  in priority order, only until their time covers the transfer's, and holds
  the rest back for later steps.  Priority: blocks of rows whose partial
  must be sent first, rows with fewer blocks left first, then Q slot, then
  KV slot (a row is finished before the next is started).  A step without a transfer (every receive done, no send ready)
  computes up to the completion of the next row that must be sent, or, with
  no send left, everything that remains.
* ``delay=False`` gives the eager variant (every ready block at once) that
  rule 2 improves on; it is used to show the rule's effect.

Also here: an exhaustive search for the optimal makespan of the same step
model (every transfer order and every split of the blocks over the steps),
usable on meshes up to 3 x 3.
"""

import functools
import math

from .block_list import DIAG, FULL, SKIP, block_list_ref

NONE, RECV_Q, RECV_KV, SEND_O = 0, 1, 2, 3


def _tile(R, C, r, c, causal, kv_rotate):
    blocks = block_list_ref(R, C, r, c, causal, kv_rotate)
    q_part = {b[0]: b[2] for b in blocks}
    kv_part = {b[1]: b[3] for b in blocks}
    need = [b for b in blocks if b[4] != SKIP]
    return blocks, q_part, kv_part, need


def _comm_time(op, costs):
    kind = op[0]
    if kind == RECV_Q:
        return costs["recv_q_s"]
    if kind == RECV_KV:
        return costs["recv_kv_s"]
    if kind == SEND_O:
        return costs["send_o_s"]
    return 0.0


def _block_time(b, costs):
    return costs["full_block_s"] if b[4] == FULL else costs["diag_block_s"]


def greedy_plan_ref(R, C, r, c, causal, kv_rotate, costs, delay=True):
    """The greedy schedule.  costs: dict with recv_q_s, recv_kv_s, send_o_s,
    full_block_s, diag_block_s (seconds).  Returns a list of steps, each a
    dict: comm (NONE / RECV_Q / RECV_KV / SEND_O), slot (-1 for NONE),
    blocks (tuples as in the block list, in compute order), comm_s,
    compute_s, start_s, end_s."""
    _, q_part, kv_part, need = _tile(R, C, r, c, causal, kv_rotate)
    g = r * C + c
    q_present = {s: q_part[s] == g for s in q_part}
    kv_present = {j: kv_part[j] == g for j in kv_part}
    rows_needed = sorted({b[0] for b in need})
    cols_needed = sorted({b[1] for b in need})
    pending = [(RECV_KV, j) for j in cols_needed if not kv_present[j]] + \
              [(RECV_Q, s) for s in rows_needed if not q_present[s]]
    sends = [s for s in rows_needed if q_part[s] != g]
    done = set()                       # computed blocks, as (q_slot, kv_slot)

    def row_left(s):
        return sum(1 for b in need if b[0] == s and (b[0], b[1]) not in done)

    def unlocks(op):
        kind, slot = op
        if kind == RECV_KV:
            return sum(1 for b in need if b[1] == slot and q_present[b[0]])
        return sum(1 for b in need if b[0] == slot and kv_present[b[1]])

    def potential(op):
        kind, slot = op
        return sum(1 for b in need if (b[1] if kind == RECV_KV else b[0]) == slot)

    steps, t = [], 0.0
    while pending or sends or len(done) < len(need):
        ready_sends = [s for s in sends if row_left(s) == 0]
        op = (NONE, -1)
        if pending:
            best = min(pending, key=lambda o: (-unlocks(o), -potential(o),
                                               0 if o[0] == RECV_Q else 1, o[1]))
            if unlocks(best) == 0 and ready_sends:
                op = (SEND_O, ready_sends[0])
            else:
                op = best
        elif ready_sends:
            op = (SEND_O, ready_sends[0])
        comm_s = _comm_time(op, costs)

        ready = [b for b in need if (b[0], b[1]) not in done and q_present[b[0]] and kv_present[b[1]]]
        ready.sort(key=lambda b: (0 if q_part[b[0]] != g else 1, row_left(b[0]), b[0], b[1]))
        chosen = []
        if not delay:
            chosen = ready
        elif op[0] != NONE:
            acc = 0.0
            for b in ready:
                if acc >= comm_s:
                    break
                chosen.append(b)
                acc += _block_time(b, costs)
        elif sends:
            # No transfer possible: compute until the next row to send is complete.
            target = ready[0][0] if ready else None
            for b in ready:
                chosen.append(b)
                if b[0] == target and all((x[0], x[1]) in done or x in chosen
                                          for x in need if x[0] == target):
                    break
        else:
            chosen = ready
        compute_s = 0.0
        for b in chosen:
            compute_s += _block_time(b, costs)
        dur = max(comm_s, compute_s)
        steps.append({"comm": op[0], "slot": op[1], "blocks": list(chosen), "comm_s": comm_s,
                      "compute_s": compute_s, "start_s": t, "end_s": t + dur})
        t += dur
        for b in chosen:
            done.add((b[0], b[1]))
        if op[0] == RECV_KV:
            kv_present[op[1]] = True
            pending.remove(op)
        elif op[0] == RECV_Q:
            q_present[op[1]] = True
            pending.remove(op)
        elif op[0] == SEND_O:
            sends.remove(op[1])
        if op[0] == NONE and not chosen:
            raise RuntimeError("schedule made no progress")
    return steps


def plan_makespan_ref(steps):
    """Sum of the step durations: max(transfer, compute) per step."""
    return math.fsum(max(s["comm_s"], s["compute_s"]) for s in steps)


def optimal_makespan_ref(R, C, r, c, causal, kv_rotate, costs):
    """Smallest makespan over every schedule of the same step model: any
    order of the transfers (receives, and sends of rows already computed),
    steps without a transfer allowed, and any split of the ready blocks over
    the steps.  Exhaustive (memoised over the set of finished transfers and
    the set of computed blocks); meant for meshes up to 3 x 3."""
    if R * C > 9:
        raise ValueError("exhaustive search is for meshes of at most 9 GPUs")
    _, q_part, kv_part, need = _tile(R, C, r, c, causal, kv_rotate)
    g = r * C + c
    ops = [(RECV_KV, j) for j in sorted({b[1] for b in need}) if kv_part[j] != g] + \
          [(RECV_Q, s) for s in sorted({b[0] for b in need}) if q_part[s] != g] + \
          [(SEND_O, s) for s in sorted({b[0] for b in need}) if q_part[s] != g]
    nb = len(need)
    all_blocks = (1 << nb) - 1
    all_ops = (1 << len(ops)) - 1
    times = [_block_time(b, costs) for b in need]

    def present(done_ops):
        qp = {s: q_part[s] == g for s in q_part}
        kp = {j: kv_part[j] == g for j in kv_part}
        for i, (kind, slot) in enumerate(ops):
            if done_ops >> i & 1:
                if kind == RECV_Q:
                    qp[slot] = True
                elif kind == RECV_KV:
                    kp[slot] = True
        return qp, kp

    @functools.lru_cache(maxsize=None)
    def best(done_ops, comp):
        if done_ops == all_ops and comp == all_blocks:
            return 0.0
        qp, kp = present(done_ops)
        avail = [i for i, b in enumerate(need) if not comp >> i & 1 and qp[b[0]] and kp[b[1]]]
        choices = [None]
        for i, (kind, slot) in enumerate(ops):
            if done_ops >> i & 1:
                continue
            if kind == SEND_O:
                row = [k for k, b in enumerate(need) if b[0] == slot]
                if not all(comp >> k & 1 for k in row):
                    continue
            choices.append(i)
        res = math.inf
        for ci in choices:
            comm_s = 0.0 if ci is None else _comm_time(ops[ci], costs)
            nd = done_ops if ci is None else done_ops | (1 << ci)
            for m in range(1 << len(avail)):
                if ci is None and m == 0:
                    continue
                mask, work = 0, 0.0
                for k, i in enumerate(avail):
                    if m >> k & 1:
                        mask |= 1 << i
                        work += times[i]
                res = min(res, max(comm_s, work) + best(nd, comp | mask))
        return res

    return best(0, 0)
